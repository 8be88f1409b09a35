"""Pins of the oracle's key blocking (CPU only).

``oracle.decode_attention`` gathers the keys of one (sequence, KV head) in blocks of at most
``chunk`` tokens (``oracle.attention.key_blocks``) and merges the blocks' (max, sum, output)
triples with the LSE rule.  Contexts up to ``KEY_BLOCK`` keys are one block; the 1M-token GPU
test is judged against the merged branch.  These tests run that branch with block sizes from 1
key up, on every format, with windows, a softcap and ALiBi, and hold it to the 40-digit
``decimal`` brute force and to the one-block result.  Planted mistakes (a key dropped or
repeated at every block boundary) must fail them.
"""
import numpy as np
import pytest

import kvgen
import oracle
import oracle.attention as oa
from oracle.brute import brute_decode_attention
from conftest import brute_as_array, oracle_args

ONE_BLOCK = 1 << 20
BLOCKS = (1, 7, 16, 513)


def _slopes(h):
    return (2.0 ** (-8.0 * (np.arange(h) + 1) / h)).astype(np.float32)


def _inputs(fmt):
    """Two ragged sequences, one of them windowed; GQA for the cheap formats.  The rotated
    codebook formats are kept short (their brute force rotates every key in 40-digit
    arithmetic)."""
    if fmt in ("bf16", "fp8"):
        return kvgen.make_inputs(kvgen.spec(
            "c1", fmt=fmt, head_dim=64, num_seqs=2, num_q_heads=4, num_kv_heads=2, context=None,
            ctx_range=(150, 300), window=200, window_frac=0.5,
            softcap=3.0 if fmt == "bf16" else 0.0), lengths=[300, 233], windows=[200, 0])
    return kvgen.make_inputs(kvgen.spec(
        "c1", fmt=fmt, head_dim=128, num_seqs=2, num_q_heads=2, num_kv_heads=1, context=None,
        ctx_range=(40, 90)), lengths=[90, 61], windows=[50, 0])


@pytest.mark.parametrize("lo,hi,block", [(0, 0, 5), (0, 1, 1), (3, 300, 7), (0, 512, 512),
                                         (5, 518, 512), (904, 5000, 1000), (0, 65536, 65536),
                                         (0, 65537, 65536)])
def test_key_blocks_tile_the_range(lo, hi, block):
    bl = oa.key_blocks(lo, hi, block)
    keys = [j for t0, t1 in bl for j in range(t0, t1)]
    assert keys == list(range(lo, hi))
    assert all(0 < t1 - t0 <= block for t0, t1 in bl)
    assert len(bl) == -(-(hi - lo) // block)


@pytest.mark.parametrize("fmt", kvgen.FORMATS)
def test_blocked_oracle_matches_brute_force(fmt):
    """Every block size gives the brute-force result to 1e-12, and the one-block result."""
    inp = _inputs(fmt)
    sl = _slopes(inp.spec.num_q_heads)
    want = brute_as_array(brute_decode_attention(*oracle_args(inp), alibi=sl))
    whole = oracle.decode_attention(*oracle_args(inp), alibi=sl, chunk=ONE_BLOCK)
    assert np.isfinite(whole).all()
    assert np.abs(whole - want).max() <= 1e-12
    for c in BLOCKS:
        got = oracle.decode_attention(*oracle_args(inp), alibi=sl, chunk=c)
        assert np.abs(got - want).max() <= 1e-12, (fmt, c)
        assert np.abs(got - whole).max() <= 1e-12, (fmt, c)


@pytest.mark.parametrize("fmt", kvgen.FORMATS)
def test_long_context_blocks_match_one_block(fmt):
    """About 9,000 keys (more than the 8,192-key blocks the oracle used to take by default),
    one sequence windowed: blocks of 1,000 and 8,192 keys and the default give the one-block
    result to 1e-12."""
    inp = kvgen.make_inputs(kvgen.spec(
        "c4", fmt=fmt, num_seqs=2, num_q_heads=2, num_kv_heads=1, context=None,
        ctx_range=(8000, 9100), pool_spare=4), lengths=[9100, 8300], windows=[8500, 0])
    sl = _slopes(2)
    whole = oracle.decode_attention(*oracle_args(inp), alibi=sl, chunk=ONE_BLOCK)
    assert np.isfinite(whole).all()
    for c in (1000, 8192, oa.KEY_BLOCK):
        got = oracle.decode_attention(*oracle_args(inp), alibi=sl, chunk=c)
        assert np.abs(got - whole).max() <= 1e-12, (fmt, c)


def test_default_block_holds_64k_keys():
    """The default keeps every context up to 64K keys in one block (no merge)."""
    assert oa.KEY_BLOCK == 65536
    assert oa.key_blocks(0, 65536, oa.KEY_BLOCK) == [(0, 65536)]


# --------------------------------------------------------------------------------------------
# planted mistakes at the block boundaries
# --------------------------------------------------------------------------------------------
def _dropped_last_key(lo, hi, block):   # one key lost at the end of every full block
    return [(t0, min(hi, t0 + block - 1)) for t0 in range(lo, hi, block)]


def _repeated_key(lo, hi, block):       # the first key of the next block counted twice
    return [(t0, min(hi, t0 + block + 1)) for t0 in range(lo, hi, block)]


@pytest.mark.parametrize("bad", [_dropped_last_key, _repeated_key])
def test_planted_block_boundary_mistakes_are_caught(monkeypatch, bad):
    inp = _inputs("bf16")
    sl = _slopes(4)
    want = brute_as_array(brute_decode_attention(*oracle_args(inp), alibi=sl))
    monkeypatch.setattr(oa, "key_blocks", bad)
    got = oracle.decode_attention(*oracle_args(inp), alibi=sl, chunk=7)
    assert np.abs(got - want).max() > 1e-6
    long_inp = kvgen.make_inputs(kvgen.spec(
        "c4", fmt="fp8", num_seqs=1, num_q_heads=2, num_kv_heads=1, context=9100, pool_spare=4))
    one = oracle.decode_attention(*oracle_args(long_inp), chunk=ONE_BLOCK)
    blocked = oracle.decode_attention(*oracle_args(long_inp), chunk=8192)
    assert np.abs(one - blocked).max() > 1e-7
