import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def oracle_args(inp, window=True):
    """Positional arguments of oracle.decode_attention for a kvgen.Inputs batch."""
    s = inp.spec
    return (inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.context_lens, s.fmt,
            inp.scales, inp.codebook, inp.sign, inp.softmax_scale,
            inp.window if window else None, inp.softcap, s.num_kv_heads, s.head_dim)


def brute_as_array(rows):
    return np.array([[[float(x) for x in r] for r in seq] for seq in rows])


@pytest.fixture
def rng():
    return np.random.default_rng(1234)
