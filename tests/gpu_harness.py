"""Run a kvgen batch through the HIP library (via the ctypes binding) and compare with the oracle."""
import json
import os

import numpy as np

import kvgen
from kvgen.torch_io import dims_kwargs, to_torch

ABS_TOL = 2e-3     # max |gpu - oracle|
REL_TOL = 1e-2     # max over rows of max_d |gpu - oracle| / max_d |oracle|


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
    ok = ~np.isnan(ref).any(axis=-1)
    g, r = gpu[ok], ref[ok]
    if g.size == 0:
        return 0.0, 0.0
    diff = np.abs(g - r)
    den = np.maximum(np.abs(r).max(axis=-1), 1e-30)
    return float(diff.max()), float((diff.max(axis=-1) / den).max())


def assert_close(gpu, ref, what=""):
    ok = ~np.isnan(ref).any(axis=-1)
    assert np.isfinite(gpu[ok]).all(), f"{what}: non-finite GPU output"
    ea, er = errors(gpu, ref)
    print(f"[parity] {what}: max_abs={ea:.3e} max_rel={er:.3e}", flush=True)
    log = os.environ.get("KVD_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(json.dumps({"case": what, "max_abs": ea, "max_rel": er}) + "\n")
    assert ea <= ABS_TOL and er <= REL_TOL, (what, ea, er)
    return ea, er
