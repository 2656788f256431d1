import json
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running case")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def golden_arrays(g, rows=None):
    """Dense q / kcache / page_table / pos arrays of a golden fixture."""
    H, D, cr, P = g["heads"], g["head_dim"], g["compress_ratio"], g["page_size"]
    kpp = P // cr
    pos = np.asarray(g["pos"], dtype=np.int32)
    R = len(pos)
    q = np.zeros((R, H, D), dtype=np.float16)
    for h, d, v in g["q_nonzero_all_rows"]:
        q[:, h, d] = v
    pt = np.asarray(g["page_table"], dtype=np.int32)
    kc = np.zeros((g["num_pages"], kpp, D), dtype=np.float16)
    for j, d, v in g["key_nonzero_logical"]:
        kc[pt[0, j // kpp], j % kpp, d] = v
    return q, kc, pt, pos


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle._load()
    return oracle
