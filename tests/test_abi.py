"""CPU tests of the C-ABI library: it loads, exports every function declared
in include/qsa.h, sizes workspaces, and rejects invalid arguments on the host
before touching a device (no GPU needed; no kernel is launched)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT
from paged_block_scoring_amd import qsa as Q

HEADER = os.path.join(ROOT, "include", "qsa.h")

FAKE = 0x10000  # an aligned, never-dereferenced pointer value


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    fns = header_functions()
    for name in ("qsa_score_paged", "qsa_topk_rows", "qsa_select_paged_tokens",
                 "qsa_topk_rows_workspace_size", "qsa_select_paged_tokens_workspace_size",
                 "qsa_last_error", "qsa_version"):
        assert name in fns


def test_library_exports_every_declared_symbol():
    L = Q.lib()
    for name in header_functions():
        assert hasattr(L, name), name
    assert set(header_functions()) == set(Q.EXPORTED)


def test_version_and_empty_error():
    assert "gfx950" in Q.qsa_version()
    assert Q.qsa_last_error() == ""


def test_workspace_sizes():
    assert Q.qsa_select_paged_tokens_workspace_size(0, 1, 100, 4, 64) == 0
    assert Q.qsa_select_paged_tokens_workspace_size(10, 1, 0, 4, 64) == 0
    fused = Q.qsa_select_paged_tokens_workspace_size(1616, 1, 46000, 4, 2048)
    Q.qsa_debug_force(Q.QSA_DEBUG_FORCE_TWO_PASS)
    try:
        two_pass = Q.qsa_select_paged_tokens_workspace_size(1616, 1, 46000, 4, 2048)
    finally:
        Q.qsa_debug_force(0)
    assert two_pass >= 1616 * 46000 * 4          # the materialised score matrix
    assert 0 < fused < two_pass                   # the fused arm never holds it
    # decode-like batches (one row per request) take the two-pass arm
    assert Q.qsa_select_paged_tokens_workspace_size(256, 256, 46000, 4, 2048) >= 256 * 46000 * 4
    assert Q.qsa_topk_rows_workspace_size(10, 100, 8) >= 0


def select(**over):
    a = dict(q=FAKE, kcache=FAKE, page_table=FAKE, pt_stride=16, num_pages=16, num_reqs=1, row_req=None,
             pos=FAKE, rows=8, heads=4, head_dim=128, page_size=64, cr=4, max_visible=256, k=64, flags=0,
             out=FAKE, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(over)
    st = Q.lib().qsa_select_paged_tokens(
        a["q"], a["kcache"], a["page_table"], a["pt_stride"], a["num_pages"], a["num_reqs"], a["row_req"],
        a["pos"], a["rows"], a["heads"], a["head_dim"], a["page_size"], a["cr"], a["max_visible"], a["k"],
        a["flags"], a["out"], a["ws"], a["ws_bytes"], a["stream"])
    return st, Q.qsa_last_error()


def score(**over):
    a = dict(q=FAKE, kcache=FAKE, page_table=FAKE, pt_stride=16, num_pages=16, num_reqs=1, row_req=None,
             pos=FAKE, rows=8, heads=4, head_dim=128, page_size=64, cr=4, max_visible=256, flags=0,
             scores=FAKE, ld=256, stream=None)
    a.update(over)
    st = Q.lib().qsa_score_paged(
        a["q"], a["kcache"], a["page_table"], a["pt_stride"], a["num_pages"], a["num_reqs"], a["row_req"],
        a["pos"], a["rows"], a["heads"], a["head_dim"], a["page_size"], a["cr"], a["max_visible"],
        a["flags"], a["scores"], a["ld"], a["stream"])
    return st, Q.qsa_last_error()


def topk(**over):
    a = dict(scores=FAKE, ld=100, visible=None, rows=4, max_visible=100, k=8, out=FAKE, ws=None, ws_bytes=0,
             stream=None)
    a.update(over)
    st = Q.lib().qsa_topk_rows(a["scores"], a["ld"], a["visible"], a["rows"], a["max_visible"], a["k"],
                               a["out"], a["ws"], a["ws_bytes"], a["stream"])
    return st, Q.qsa_last_error()


@pytest.mark.parametrize("over,code", [
    (dict(heads=3), Q.QSA_ERR_UNSUPPORTED),
    (dict(head_dim=64), Q.QSA_ERR_UNSUPPORTED),
    (dict(k=63), Q.QSA_ERR_INVALID_ARGUMENT),                 # k not a multiple of cr
    (dict(k=0), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(k=4 * (Q.QSA_MAX_SELECT + 1)), Q.QSA_ERR_UNSUPPORTED),
    (dict(k=Q.QSA_MAX_SELECT + 1, flags=Q.QSA_OUT_KEYS), Q.QSA_ERR_UNSUPPORTED),
    (dict(q=None), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(kcache=None), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(page_table=None), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(pos=None), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(out=None), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(ws=None), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(ws_bytes=16), Q.QSA_ERR_WORKSPACE_TOO_SMALL),
    (dict(page_size=66), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(cr=0), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(pt_stride=15), Q.QSA_ERR_INVALID_ARGUMENT),        # 256 keys need 16 pages of 16 keys
    (dict(num_pages=0), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(num_reqs=0), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(rows=-1), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(max_visible=-1), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(flags=0x10), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(q=FAKE + 4), Q.QSA_ERR_INVALID_ARGUMENT),           # misaligned
])
def test_select_rejects_before_device(over, code):
    st, msg = select(**over)
    assert st == code, msg
    assert re.match(r"^qsa_api\.hip:\d+: .+", msg), msg


@pytest.mark.parametrize("over,code", [
    (dict(ld=255), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(scores=None), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(flags=Q.QSA_OUT_KEYS), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(heads=8), Q.QSA_ERR_UNSUPPORTED),
])
def test_score_rejects_before_device(over, code):
    st, msg = score(**over)
    assert st == code, msg


@pytest.mark.parametrize("over,code", [
    (dict(k=0), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(k=Q.QSA_MAX_SELECT + 1), Q.QSA_ERR_UNSUPPORTED),
    (dict(ld=99), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(out=None), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(rows=-2), Q.QSA_ERR_INVALID_ARGUMENT),
])
def test_topk_rejects_before_device(over, code):
    st, msg = topk(**over)
    assert st == code, msg


def test_zero_rows_is_a_noop_without_device():
    assert select(rows=0, q=None, out=None, ws=None, ws_bytes=0)[0] == Q.QSA_OK
    assert score(rows=0, q=None, scores=None)[0] == Q.QSA_OK
    assert topk(rows=0, out=None)[0] == Q.QSA_OK


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros((2, 4, 128), dtype=torch.float16)
    kc = torch.zeros((3, 16, 128), dtype=torch.float16)
    with pytest.raises(ValueError, match="device tensor"):
        Q.qsa_select_paged_tokens(q, kc, torch.zeros((1, 1), dtype=torch.int32), torch.zeros(2, dtype=torch.int32),
                                  4, 64, max_visible=1)


def _host_paged():
    import torch
    return dict(q=torch.zeros((2, 4, 128), dtype=torch.float16), kcache=torch.zeros((3, 16, 128), dtype=torch.float16),
                page_table=torch.zeros((1, 3), dtype=torch.int32), pos=torch.zeros(2, dtype=torch.int32))


def test_binding_requires_max_visible():
    """The binding computes nothing: the visible-key bound is the caller's."""
    a = _host_paged()
    with pytest.raises(TypeError):
        Q.qsa_select_paged_tokens(a["q"], a["kcache"], a["page_table"], a["pos"], 4, 64)
    with pytest.raises(TypeError):
        Q.qsa_score_paged(a["q"], a["kcache"], a["page_table"], a["pos"], 4)


def test_binding_refuses_mis_shaped_tensors_before_any_call():
    """Shape relations are checked before the device check, so these fail on
    the host with a shape message; the library is never called."""
    import torch
    a = _host_paged()
    with pytest.raises(ValueError, match="head_dim"):
        Q.qsa_select_paged_tokens(a["q"], torch.zeros((3, 16, 64), dtype=torch.float16), a["page_table"], a["pos"],
                                  4, 64, max_visible=1)
    with pytest.raises(ValueError, match="shape"):
        Q.qsa_select_paged_tokens(a["q"], a["kcache"], a["page_table"], a["pos"], 4, 64, max_visible=1,
                                  out=torch.zeros((2, 32), dtype=torch.int32))
    with pytest.raises(ValueError, match="shape"):
        Q.qsa_score_paged(a["q"], a["kcache"], a["page_table"], a["pos"], 4, max_visible=5,
                          scores=torch.zeros((2, 4), dtype=torch.float32))
    with pytest.raises(ValueError, match="shape"):
        Q.qsa_topk_rows(torch.zeros((3, 10), dtype=torch.float32), 4, out=torch.zeros((3, 5), dtype=torch.int32))
    with pytest.raises(ValueError, match="shape"):
        Q.qsa_sparse_attention(torch.zeros((2, 24, 256), dtype=torch.float16),
                               torch.zeros((1, 64, 2, 256), dtype=torch.float16),
                               torch.zeros((1, 64, 2, 256), dtype=torch.float16), a["page_table"],
                               torch.zeros((2, 8), dtype=torch.int32), out=torch.zeros((2, 24, 128)))
    Q.qsa_last_error()  # nothing was called: no error is pending from these


def test_debug_force_rejects_bad_masks():
    assert Q.qsa_debug_forced() == 0
    for bad in (0x80, Q.QSA_DEBUG_FORCE_TWO_PASS | Q.QSA_DEBUG_FORCE_FUSED,
                Q.QSA_DEBUG_FORCE_TWO_PASS | Q.QSA_DEBUG_FORCE_FALLBACK,
                Q.QSA_DEBUG_FORCE_TWO_PASS | Q.QSA_DEBUG_FORCE_REDO,
                Q.QSA_DEBUG_FORCE_STREAM | Q.QSA_DEBUG_FORCE_TWO_PASS,
                Q.QSA_DEBUG_FORCE_STREAM | Q.QSA_DEBUG_FORCE_FUSED,
                Q.QSA_DEBUG_FORCE_STREAM | Q.QSA_DEBUG_FORCE_REDO,
                Q.QSA_DEBUG_FORCE_TILES | Q.QSA_DEBUG_FORCE_GROUPS):
        with pytest.raises(Q.QSAError) as e:
            Q.qsa_debug_force(bad)
        assert e.value.status == Q.QSA_ERR_INVALID_ARGUMENT
        assert Q.qsa_debug_forced() == 0
    Q.qsa_debug_force(Q.QSA_DEBUG_FORCE_FALLBACK | Q.QSA_DEBUG_FORCE_GROUPS)
    try:
        assert Q.qsa_debug_forced() == Q.QSA_DEBUG_FORCE_FALLBACK | Q.QSA_DEBUG_FORCE_GROUPS
        # the workspace query follows the forced arm: a decode batch now sizes the fused arm
        fused = Q.qsa_select_paged_tokens_workspace_size(256, 256, 46000, 4, 2048)
    finally:
        Q.qsa_debug_force(0)
    assert 0 < fused < Q.qsa_select_paged_tokens_workspace_size(256, 256, 46000, 4, 2048)
    Q.qsa_debug_force(Q.QSA_DEBUG_FORCE_REDO)
    try:  # the redo override also drives the fused arm
        assert Q.qsa_select_paged_tokens_workspace_size(256, 256, 46000, 4, 2048) == fused
    finally:
        Q.qsa_debug_force(0)
    Q.qsa_debug_force(Q.QSA_DEBUG_FORCE_STREAM)
    try:  # streaming arm: 6 chunk lists of 512 composites (8 bytes) per row, then 6 counts
        stream = Q.qsa_select_paged_tokens_workspace_size(256, 256, 46000, 4, 2048)
    finally:
        Q.qsa_debug_force(0)
    assert stream == 256 * 6 * 512 * 8 + 256 * 6 * 4
    # the caller's flag asks for the same arm, and the workspace follows it
    assert Q.qsa_select_paged_tokens_workspace_size(256, 256, 46000, 4, 2048, Q.QSA_STREAM_SELECT) == stream
    Q.qsa_debug_force(Q.QSA_DEBUG_FORCE_TWO_PASS)
    try:  # a forced arm overrides the flag
        assert (Q.qsa_select_paged_tokens_workspace_size(256, 256, 46000, 4, 2048, Q.QSA_STREAM_SELECT)
                == Q.qsa_select_paged_tokens_workspace_size(256, 256, 46000, 4, 2048))
    finally:
        Q.qsa_debug_force(0)


def attend(**over):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, page_table=FAKE, pt_stride=16, num_pages=16, num_reqs=1, row_req=None,
             tokens=FAKE, k=2048, rows=8, q_heads=24, kv_heads=2, head_dim=256, page_size=64, scale=0.0625,
             out=FAKE, workspace=FAKE, workspace_bytes=1 << 30, stream=None)
    a.update(over)
    st = Q.lib().qsa_sparse_attention(
        a["q"], a["kc"], a["vc"], a["page_table"], a["pt_stride"], a["num_pages"], a["num_reqs"], a["row_req"],
        a["tokens"], a["k"], a["rows"], a["q_heads"], a["kv_heads"], a["head_dim"], a["page_size"], a["scale"],
        a["out"], a["workspace"], a["workspace_bytes"], a["stream"])
    return st, Q.qsa_last_error()


@pytest.mark.parametrize("over,code", [
    (dict(head_dim=128), Q.QSA_ERR_UNSUPPORTED),
    (dict(q_heads=25), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(q_heads=34, kv_heads=2), Q.QSA_ERR_UNSUPPORTED),     # 17 query heads per KV head
    (dict(kv_heads=0), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(k=0), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(rows=-1), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(page_size=0), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(num_pages=0), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(num_reqs=0), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(pt_stride=0), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(num_pages=1 << 30), Q.QSA_ERR_UNSUPPORTED),          # rows of the cache past 2^32
    (dict(scale=float("inf")), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(tokens=None), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(vc=None), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(out=None), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(q=FAKE + 4), Q.QSA_ERR_INVALID_ARGUMENT),            # misaligned
    (dict(workspace_bytes=1000), Q.QSA_ERR_WORKSPACE_TOO_SMALL),  # 8 rows split over several workgroups
    (dict(workspace=None), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(workspace=FAKE + 8), Q.QSA_ERR_INVALID_ARGUMENT),    # misaligned
])
def test_attention_rejects_before_device(over, code):
    st, msg = attend(**over)
    assert st == code, msg
    assert re.match(r"^qsa_api\.hip:\d+: .+", msg), msg


def test_attention_zero_rows_is_a_noop():
    st, msg = attend(rows=0, q=None, kc=None, vc=None, page_table=None, tokens=None, out=None)
    assert st == Q.QSA_OK, msg


def compress(**over):
    a = dict(k_tok=FAKE, tok_req=None, tok_pos=FAKE, tokens=64, head_dim=128, norm_w=None, eps=1e-6, rope_dim=128,
             rope_base=10000.0, flags=0, state=FAKE, kcache=FAKE, page_table=FAKE, pt_stride=16, num_pages=16,
             num_reqs=1, page_size=64, compress_ratio=4, stream=None)
    a.update(over)
    st = Q.lib().qsa_compress_keys(
        a["k_tok"], a["tok_req"], a["tok_pos"], a["tokens"], a["head_dim"], a["norm_w"], a["eps"], a["rope_dim"],
        a["rope_base"], a["flags"], a["state"], a["kcache"], a["page_table"], a["pt_stride"], a["num_pages"],
        a["num_reqs"], a["page_size"], a["compress_ratio"], a["stream"])
    return st, Q.qsa_last_error()


@pytest.mark.parametrize("over,code", [
    (dict(tokens=-1), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(head_dim=256), Q.QSA_ERR_UNSUPPORTED),
    (dict(compress_ratio=0), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(compress_ratio=128, page_size=128), Q.QSA_ERR_UNSUPPORTED),
    (dict(page_size=66), Q.QSA_ERR_INVALID_ARGUMENT),           # not a multiple of the ratio
    (dict(page_size=2), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(rope_dim=-16), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(rope_dim=144), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(rope_dim=40), Q.QSA_ERR_UNSUPPORTED),
    (dict(rope_base=0.0), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(rope_base=float("nan")), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(eps=-1.0), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(eps=float("inf")), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(flags=0x1), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(num_pages=0), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(num_reqs=0), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(pt_stride=0), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(k_tok=None), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(kcache=None), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(state=None), Q.QSA_ERR_INVALID_ARGUMENT),
    (dict(state=FAKE + 2), Q.QSA_ERR_INVALID_ARGUMENT),         # misaligned
])
def test_compress_rejects_before_device(over, code):
    st, msg = compress(**over)
    assert st == code, msg
    assert re.match(r"^qsa_api\.hip:\d+: .+", msg), msg


def test_compress_edge_arguments_pass_the_host_checks():
    # no tokens: nothing to do, no pointer is looked at
    st, msg = compress(tokens=0, k_tok=None, tok_pos=None, kcache=None, page_table=None, state=None)
    assert st == Q.QSA_OK, msg
    # rope_dim 0 ignores the base
    st, msg = compress(tokens=0, rope_dim=0, rope_base=0.0)
    assert st == Q.QSA_OK, msg


def test_attention_workspace_sizes():
    ws = Q.qsa_sparse_attention_workspace_size
    # 256 rows x 2 KV heads fill the device: no split, no workspace
    assert ws(256, 24, 2, 256, 2048) == 0
    assert ws(2000, 24, 2, 256, 2048) == 0
    # few rows: each (row, KV head) splits its list; one record per split
    one = ws(1, 24, 2, 256, 2048)
    eight = ws(8, 24, 2, 256, 2048)
    assert one > 0 and eight > 0
    assert eight % (8 * 2) == 0 and one % 2 == 0
    # lists are not split below 128 entries per split
    assert ws(1, 24, 2, 256, 100) == 0
    assert ws(1, 24, 2, 256, 256) == 2 * 2 * (32 + 16 * 256) * 4
    # unsupported shapes need nothing
    assert ws(1, 24, 2, 128, 2048) == 0
    assert ws(0, 24, 2, 256, 2048) == 0
    # a large enough workspace passes the host checks (zero rows: nothing runs)
    st, msg = attend(rows=0, workspace_bytes=eight)
    assert st == Q.QSA_OK, msg


def test_binding_refuses_host_tensors_and_bad_shapes_for_the_adjacent_steps():
    import torch
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32)  # noqa: E731
    f16 = lambda *s: torch.zeros(s, dtype=torch.float16)  # noqa: E731
    # producer: host tensors are refused before the library is called
    with pytest.raises(ValueError):
        Q.qsa_compress_keys(f16(8, 128), i32(8), f16(1, 4, 128), f16(4, 16, 128), i32(1, 4), 4)
    # wrong dtype
    with pytest.raises(TypeError):
        Q.qsa_compress_keys(torch.zeros((8, 128)), i32(8), f16(1, 4, 128), f16(4, 16, 128), i32(1, 4), 4)
    # consumer: host tensors refused
    with pytest.raises(ValueError):
        Q.qsa_sparse_attention(f16(2, 24, 256), f16(4, 64, 2, 256), f16(4, 64, 2, 256), i32(1, 4), i32(2, 16))
    with pytest.raises(TypeError):
        Q.qsa_sparse_attention(torch.zeros((2, 24, 256)), f16(4, 64, 2, 256), f16(4, 64, 2, 256), i32(1, 4),
                               i32(2, 16))


def test_noalloc_rejects_calls_beyond_its_scratch():
    """A call whose workspace would exceed the static scratch is refused on
    the host, naming both sizes, before any device call."""
    need = Q.qsa_select_paged_tokens_workspace_size(4096, 1, 200000, 4, 2048)
    assert need > Q.QSA_NOALLOC_SCRATCH_BYTES
    st = Q.lib().qsa_select_paged_tokens_noalloc(FAKE, FAKE, FAKE, 12500, 20000, 1, None, FAKE, 4096, 4, 128, 64,
                                                 4, 200000, 2048, 0, FAKE, None)
    assert st == Q.QSA_ERR_UNSUPPORTED
    msg = Q.qsa_last_error()
    assert str(need) in msg and str(Q.QSA_NOALLOC_SCRATCH_BYTES) in msg
    # argument errors come first, as in the workspace entry point
    st = Q.lib().qsa_select_paged_tokens_noalloc(FAKE, FAKE, FAKE, 12500, 20000, 1, None, FAKE, 4096, 5, 128, 64,
                                                 4, 200000, 2048, 0, FAKE, None)
    assert st == Q.QSA_ERR_UNSUPPORTED and "heads" in Q.qsa_last_error()
    assert Q.lib().qsa_select_paged_tokens_noalloc(None, None, None, 1, 1, 1, None, None, 0, 4, 128, 64, 4, 0, 64,
                                                   0, None, None) == Q.QSA_OK
