"""GPU parity of the KV append (quantize-on-write) kernel: the caches and per-token norms it
writes equal the oracle's cache writer byte for byte (oracle/encode.py), for every format, for
decode-step and multi-token appends crossing pages, ragged positions, skipped tokens, values
that saturate FP8, NaN inputs and zero vectors; and attention over the appended cache matches
the oracle."""
import numpy as np
import pytest

import kvgen
import oracle
from oracle import encode as enc
from conftest import oracle_args
from gpu_harness import GpuBatch, assert_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _append_case(fmt, old_lengths, T, seed, d=128, hkv=2, mutate=None):
    """A cache holding old_lengths tokens per sequence plus pages for T more; returns the
    batch, the new tokens, the positions and the (block table, k, v, scales) after both the
    GPU and the oracle appended them."""
    import torch
    import quantized_kv_cache_split_amd as kvd
    from kvgen.torch_io import dims_kwargs, to_torch

    B = len(old_lengths)
    s = kvgen.spec("c1", fmt=fmt, head_dim=d, num_q_heads=2 * hkv, num_kv_heads=hkv,
                   pool_total=None, num_seqs=B, seed=seed)
    inp = kvgen.make_inputs(s, lengths=[L + T for L in old_lengths])
    rng = np.random.default_rng(seed + 100)
    kn = rng.standard_normal((B, T, hkv, d)).astype(np.float32)
    vn = rng.standard_normal((B, T, hkv, d)).astype(np.float32)
    pos = np.array(old_lengths, dtype=np.int32)
    bt = inp.block_table.copy()
    if mutate:
        mutate(kn, vn, pos, bt, inp)
    inp.block_table = bt
    t = to_torch(inp, "cuda:0")
    dims = kvd.Dims(**dims_kwargs(inp, 0))
    kg = torch.from_numpy(kn).to("cuda:0")
    vg = torch.from_numpy(vn).to("cuda:0")
    pg = torch.from_numpy(pos).to("cuda:0")
    kvd.append_kv(dims, fmt, kg, vg, t["block_table"], pg, T, t["k_cache"], t["v_cache"],
                  t["scales"], t["codebook"], t["sign_pattern"])
    torch.cuda.synchronize()
    gpu = (t["k_cache"].cpu().numpy(), t["v_cache"].cpu().numpy(),
           None if t["scales"] is None else t["scales"].cpu().numpy())
    ref = enc.append_tokens(fmt, kn, vn, bt, pos, inp.k_cache, inp.v_cache, inp.scales,
                            inp.codebook, inp.sign)
    return inp, gpu, ref


def _assert_same(gpu, ref, what):
    for name, g, r in zip(("k_cache", "v_cache", "scales"), gpu, ref):
        if r is None:
            continue
        g8 = np.ascontiguousarray(g).view(np.uint8)
        r8 = np.ascontiguousarray(r).view(np.uint8)
        bad = np.flatnonzero(g8.reshape(-1) != r8.reshape(-1))
        assert bad.size == 0, f"{what} {name}: {bad.size} bytes differ, first at {bad[:8]}"


@pytest.mark.parametrize("fmt", kvgen.FORMATS)
@pytest.mark.parametrize("old", [[0], [15], [16], [7, 31, 100]])
def test_append_one_token(fmt, old):
    inp, gpu, ref = _append_case(fmt, old, 1, seed=3)
    _assert_same(gpu, ref, f"{fmt} T=1 old={old}")


@pytest.mark.parametrize("fmt", kvgen.FORMATS)
def test_append_many_tokens_crossing_pages(fmt):
    inp, gpu, ref = _append_case(fmt, [5, 40, 1], 37, seed=4)
    _assert_same(gpu, ref, f"{fmt} T=37")


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_append_head_dim_64(fmt):
    inp, gpu, ref = _append_case(fmt, [3, 20], 9, seed=5, d=64)
    _assert_same(gpu, ref, f"{fmt} D=64")


@pytest.mark.parametrize("fmt", kvgen.FORMATS)
def test_append_skips_tokens_without_a_page(fmt):
    def mutate(kn, vn, pos, bt, inp):
        bt[0, (pos[0] + 2) // 16] = -1                  # this page is not in the pool
        bt[1, (pos[1] + 1) // 16] = inp.num_pool_blocks + 3
        pos[2] = bt.shape[1] * 16 - 2                   # the last tokens run past the table
    inp, gpu, ref = _append_case(fmt, [4, 30, 10], 6, seed=6, mutate=mutate)
    _assert_same(gpu, ref, f"{fmt} skipped tokens")


def test_append_fp8_saturation_and_nan():
    def mutate(kn, vn, pos, bt, inp):
        kn[0, 0, 0, :8] = [1e9, -1e9, np.inf, -np.inf, np.nan, 0.0, -0.0, 1e-30]
        vn[0, 1, 1, :4] = [5e3, -5e3, np.nan, 3e-12]
    inp, gpu, ref = _append_case("fp8", [2, 9], 3, seed=7, mutate=mutate)
    _assert_same(gpu, ref, "fp8 saturation")


def test_append_turbo8_k_saturation():
    """Turbo8 K goes through the FP8 encoder with the per-head K scale stored after the V
    norms: saturation, infinities, NaN and signed zero as for FP8."""
    def mutate(kn, vn, pos, bt, inp):
        kn[0, 0, 1, :8] = [1e9, -1e9, np.inf, -np.inf, np.nan, 0.0, -0.0, 1e-30]
    inp, gpu, ref = _append_case("turbo8", [2, 9], 3, seed=11, mutate=mutate)
    _assert_same(gpu, ref, "turbo8 K saturation")


def test_append_bf16_nan_inf():
    def mutate(kn, vn, pos, bt, inp):
        kn[0, 0, 0, :4] = [np.nan, np.inf, -np.inf, 3.4e38]
    inp, gpu, ref = _append_case("bf16", [2], 2, seed=8, mutate=mutate)
    _assert_same(gpu, ref, "bf16 nan/inf")


@pytest.mark.parametrize("fmt", ["turbo4", "turbo3", "turbo8"])
def test_append_turbo_zero_and_scaled_vectors(fmt):
    def mutate(kn, vn, pos, bt, inp):
        kn[0, 0, 0] = 0.0
        vn[0, 0, 1] = 0.0
        kn[0, 1, 0] *= 1e-20
        vn[0, 1, 0] *= 1e20
    inp, gpu, ref = _append_case(fmt, [6], 4, seed=9, mutate=mutate)
    _assert_same(gpu, ref, f"{fmt} zero/scaled")


@pytest.mark.parametrize("fmt", kvgen.FORMATS)
def test_attention_over_appended_cache(fmt):
    """Append 300 tokens to 2 sequences, then decode over the result on the GPU and compare
    with the oracle on the oracle-written cache."""
    import torch
    inp, gpu, ref = _append_case(fmt, [100, 900], 300, seed=10)
    _assert_same(gpu, ref, f"{fmt} before attention")
    inp.k_cache, inp.v_cache = ref[0], ref[1]
    if ref[2] is not None:
        inp.scales = ref[2]
    assert_close(GpuBatch(inp).run(), oracle.decode_attention(*oracle_args(inp)), f"{fmt} appended")
