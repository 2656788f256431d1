"""The allocation-free entry point against the workspace one.

qsa_select_paged_tokens_noalloc runs the same kernels as
qsa_select_paged_tokens on a static per-device scratch instead of a caller
workspace.  Its output must equal the workspace entry point's, bit for bit,
on consecutive calls that reuse the scratch: the full 1,616-row x 184k
kernel shape (fused arm, the largest scratch of the benchmark workloads),
then a smaller decode batch (two-pass arm) and a tiny batch, so that a
later, smaller call meets the larger call's leftovers.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from paged_block_scoring_amd import qsa as Q

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _call_both(w, flags):
    d = {n: torch.from_numpy(getattr(w, n)).to(DEV) for n in ("q", "kcache", "page_table", "pos", "row_req")}
    mv = max(oracle.visible_keys(int(p), w.compress_ratio) for p in w.pos)
    need = Q.qsa_select_paged_tokens_workspace_size(w.rows, w.num_reqs, mv, w.compress_ratio, w.k, flags)
    assert need <= Q.QSA_NOALLOC_SCRATCH_BYTES
    ref = Q.qsa_select_paged_tokens(d["q"], d["kcache"], d["page_table"], d["pos"], w.compress_ratio, w.k,
                                    max_visible=mv, row_req=d["row_req"], flags=flags)
    path = Q.qsa_last_path()
    out = torch.full((w.rows, w.k), -7, dtype=torch.int32, device=DEV)
    Q.qsa_select_paged_tokens_noalloc(d["q"], d["kcache"], d["page_table"], d["pos"], w.compress_ratio, w.k,
                                      max_visible=mv, out=out, row_req=d["row_req"], flags=flags)
    assert Q.qsa_last_path() == path
    torch.cuda.synchronize()
    return ref.cpu().numpy(), out.cpu().numpy(), path


@pytest.mark.parametrize("flags", [0, Q.QSA_SCORE_RELU])
def test_noalloc_equals_workspace_entry_point(flags):
    paths = []
    for w in (W.kernel_shape(), W.decode(num_reqs=24), W.tiny()):
        print(f"noalloc: {w.name} rows={w.rows} flags={flags}", flush=True)
        ref, got, path = _call_both(w, flags)
        assert np.array_equal(got, ref), (w.name, flags, path)
        paths.append(path)
    assert paths[0] == "fused" and paths[1] == "two_pass"
