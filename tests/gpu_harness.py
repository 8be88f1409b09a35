"""Run a kvgen batch through the HIP library (via the ctypes binding) and compare with the oracle."""
import json
import os

import numpy as np

import kvgen
from kvgen.torch_io import dims_kwargs, to_torch

ABS_TOL = 2e-3     # max |gpu - oracle|
REL_TOL = 1e-2     # max over rows of max_d |gpu - oracle| / max_d |oracle|

# Tighter per-format bound on the row RMS-relative error ||gpu - oracle||_2 / ||oracle||_2 (max
# over rows), from the operand precision of each format's matrix products:
#   BF16, FP8: exact bf16 K / V operands, P fed as a bf16 hi + lo pair (2^-16 relative), fp32
#     accumulation -- measured at most 1.2e-5 over every GPU case (6e-6 at full sizes);
#   codebook V (Turbo4, Turbo3, Turbo8): P' and the V levels each rounded once to fp16 (2^-12
#     relative: random for P', a fixed relative error per level for V), so the output error is a
#     few 1e-4 of the row, independent of the context length and of the logits' size --
#     measured at most 4.9e-4 over every GPU case.
# At 32K keys a single dropped key of typical weight moves some row by 3e-3 to 2e-2 of its norm
# (tests/test_oracle_sensitivity.py shows this on the oracle): more than twice either bound.
ROW_RMS_TOL = {"bf16": 5e-5, "fp8": 5e-5, "turbo4": 1e-3, "turbo3": 1e-3, "turbo8": 1e-3}


def format_of(what):
    """The cache format a parity case name refers to: a format token ('turbo4 L=300') or a
    workload name ('c4 seq 3 kv head 1')."""
    for tok in str(what).replace(":", " ").replace(",", " ").split():
        if tok in kvgen.FORMATS:
            return tok
        if tok in kvgen.SPECS:
            return kvgen.SPECS[tok].fmt
    raise ValueError(f"parity case {what!r} names no cache format")


class GpuBatch:
    """Device copy of one batch plus output and workspace buffers."""

    def __init__(self, inp, partition_size=None, device="cuda:0", partitions_per_wave=0,
                 alibi=None):
        import torch
        import quantized_kv_cache_split_amd as kvd
        self.kvd = kvd
        self.inp = inp
        self.dims = kvd.Dims(**dims_kwargs(inp, partition_size, partitions_per_wave))
        self.t = to_torch(inp, device)
        self.alibi = None if alibi is None else torch.from_numpy(
            np.asarray(alibi, dtype=np.float32)).to(device)
        s = inp.spec
        self.out = torch.full(tuple(inp.q.shape), float("nan"), dtype=torch.float32,
                              device=device)
        nbytes = kvd.workspace_bytes(self.dims)
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        if nbytes:
            self.ws.view(torch.float32)[:].fill_(float("nan"))

    def _args(self, window=True):
        t, s = self.t, self.inp.spec
        return (self.dims, t["q"], t["k_cache"], t["v_cache"], t["block_table"],
                t["context_lens"], s.fmt, t["scales"], t["codebook"], t["sign_pattern"],
                float(self.inp.softmax_scale), t["window"] if window else None,
                float(self.inp.softcap), self.out, self.ws if self.kvd.workspace_bytes(self.dims) else None)

    def run(self, window=True):
        self.kvd.decode_attn_paged(*self._args(window), alibi_slopes=self.alibi)
        import torch
        torch.cuda.synchronize()
        return self.out.double().cpu().numpy()

    def run_phase1(self):
        self.kvd.decode_partitions(*self._args(), alibi_slopes=self.alibi)
        import torch
        torch.cuda.synchronize()

    def partials(self):
        """Workspace triples (m, l, o) as numpy arrays [B, Hq, P], [B, Hq, P], [B, Hq, P, D]
        (with a chunk of n_q queries: [B, n_q, Hq, P] ...)."""
        s = self.inp.spec
        B, Hq, D, nq = s.num_seqs, s.num_q_heads, s.head_dim, s.queries_per_seq
        ps = self.dims.partition_size or 512     # partitions as the header defines them
        P = -(-self.dims.max_context_len // ps)
        lead = (B, Hq) if nq == 1 else (B, nq, Hq)
        rows = B * nq * Hq * P
        ml = -(-rows * 4 // 256) * 256
        ws = self.ws.cpu().numpy()
        m = ws[:rows * 4].view(np.float32).reshape(*lead, P)
        l = ws[ml:ml + rows * 4].view(np.float32).reshape(*lead, P)
        o = ws[2 * ml:2 * ml + rows * D * 4].view(np.float32).reshape(*lead, P, D)
        return m, l, o


def errors(gpu, ref):
    """(max abs error, max row-normwise relative error) over rows where the oracle is defined."""
    ea, er, _, _ = error_stats(gpu, ref)
    return ea, er


def error_stats(gpu, ref):
    """Errors over the rows (last axis = head_dim) where the oracle is defined:
    max abs; max over rows of max_d |g - o| / max_d |o| (row-normwise, the required gate);
    max over rows of ||g - o||_2 / ||o||_2 (row RMS-relative); ||g - o||_F / ||o||_F over all
    rows (RMS-relative)."""
    ok = ~np.isnan(ref).any(axis=-1)
    g, r = gpu[ok], ref[ok]
    if g.size == 0:
        return 0.0, 0.0, 0.0, 0.0
    diff = np.abs(g - r)
    den = np.maximum(np.abs(r).max(axis=-1), 1e-30)
    row2 = np.sqrt((diff ** 2).sum(axis=-1)) / np.maximum(np.sqrt((r ** 2).sum(axis=-1)), 1e-30)
    rms = float(np.sqrt((diff ** 2).sum()) / max(float(np.sqrt((r ** 2).sum())), 1e-30))
    return float(diff.max()), float((diff.max(axis=-1) / den).max()), float(row2.max()), rms


def assert_close(gpu, ref, what=""):
    ok = ~np.isnan(ref).any(axis=-1)
    assert np.isfinite(gpu[ok]).all(), f"{what}: non-finite GPU output"
    ea, er, e2, rms = error_stats(gpu, ref)
    print(f"[parity] {what}: max_abs={ea:.3e} max_rel={er:.3e} row_rms_rel={e2:.3e} "
          f"rms_rel={rms:.3e}", flush=True)
    log = os.environ.get("KVD_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(json.dumps({"case": what, "max_abs": ea, "max_rel": er, "row_rms_rel": e2,
                                "rms_rel": rms}) + "\n")
    assert ea <= ABS_TOL and er <= REL_TOL, (what, ea, er)
    assert e2 <= ROW_RMS_TOL[format_of(what)], (what, e2)
    return ea, er


def runs_per_triple(fmt):
    """Runs whose triples the partition kernel merges into one workspace triple: the waves of
    one workgroup (4 for BF16 / FP8, 8 for the codebook formats)."""
    return 8 if fmt in ("turbo4", "turbo3", "turbo8") else 4


def _merge_group(g):
    """LSE merge of triples [(lo, hi, m, l, o), ...] (natural-log m): M = max m_i,
    l = sum l_i e^(m_i - M), o = sum l_i e^(m_i - M) o_i / l; rows with no key keep m = -inf,
    l = 0, o = 0."""
    ms = np.array([x[2] for x in g], dtype=np.float64)
    ls = np.array([x[3] for x in g], dtype=np.float64)
    os_ = np.array([x[4] for x in g], dtype=np.float64)
    M = ms.max(axis=0)
    safe = np.where(np.isfinite(M), M, 0.0)
    w = np.where(ls > 0, ls * np.exp(np.where(ls > 0, ms, 0.0) - safe), 0.0)
    L = w.sum(axis=0)
    O = np.einsum("pr,prd->rd", w, os_) / np.where(L > 0, L, 1.0)[:, None]
    return M, L, O


def merge_runs(parts, part_size, run):
    """Group an oracle's per-partition triples [(lo, hi, m, l, o), ...] (in order, natural-log
    m) into groups of ``run`` consecutive partitions the partition kernel merges into one
    workspace triple (a workgroup's runs: partitions per run x runs_per_triple; groups start
    at the first partition of the range), merging each group with the LSE rule (_merge_group).
    Returns [(slot, lo, hi, m, l, o)]: group k of a range whose first partition is p0 sits in
    workspace slot p0 + k."""
    if not parts:
        return []
    p0 = parts[0][0] // part_size
    groups = {}
    for lo, hi, m, l, o in parts:
        groups.setdefault((lo // part_size - p0) // run, []).append((lo, hi, m, l, o))
    return [(p0 + k, groups[k][0][0], groups[k][-1][1], *_merge_group(groups[k]))
            for k in sorted(groups)]


def merge_blocks(parts, starts):
    """Group an oracle's triples over short token ranges (in order, each inside one block) by
    the workgroup block holding them -- block x covers tokens [starts[x], starts[x + 1]) -- and
    merge each group (_merge_group).  Returns [(x, lo, hi, m, l, o)] for the blocks that hold
    any of the ranges."""
    groups = {}
    for lo, hi, m, l, o in parts:
        x = int(np.searchsorted(starts, lo, side="right")) - 1
        assert 0 <= x < len(starts) - 1 and hi <= starts[x + 1], (lo, hi, starts)
        groups.setdefault(x, []).append((lo, hi, m, l, o))
    return [(x, groups[x][0][0], groups[x][-1][1], *_merge_group(groups[x]))
            for x in sorted(groups)]

