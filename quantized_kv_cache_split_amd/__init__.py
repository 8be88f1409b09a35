"""Python binding of libkvdecode.so: single-query decode attention over a paged KV cache on
MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the library's HIP kernels.
Functions take torch tensors that already live on the GPU (or None for optional arguments),
pass their device pointers and the current HIP stream to the C ABI (include/kvdecode.h) and
raise KvdError on a non-zero status.  Importing this module loads the library and fails loudly
if it has not been built.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["Dims", "KvdError", "BF16", "FP8_E4M3", "TURBO4", "TURBO3", "TURBO8", "FORMATS",
           "workspace_bytes", "decode_attn_paged", "decode_attn_paged_noalloc", "decode_partitions", "reduce_partitions",
           "dequant_gather", "dequant_operands", "append_kv", "read_probe", "status_str",
           "library_path", "load",
           "hip_runtimes_mapped"]

BF16, FP8_E4M3, TURBO4, TURBO3, TURBO8 = 0, 1, 2, 3, 4
FORMATS = {"bf16": BF16, "fp8": FP8_E4M3, "turbo4": TURBO4, "turbo3": TURBO3, "turbo8": TURBO8}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkvdecode.so")
_lib = None


KVD_ERR_HIP = -6


def _hip_error() -> str:
    """Name and text of the HIP runtime's pending error on this thread (a failed launch leaves
    its error there), or '' when there is none.  Reading it clears it.  Asks the runtime already
    mapped into the process (opening one by name could load a second runtime)."""
    try:
        mapped = hip_runtimes_mapped()
        if len(mapped) != 1:
            return ""
        hip = ctypes.CDLL(mapped[0])
        hip.hipGetLastError.restype = ctypes.c_int
        hip.hipGetErrorName.argtypes = [ctypes.c_int]
        hip.hipGetErrorName.restype = ctypes.c_char_p
        hip.hipGetErrorString.argtypes = [ctypes.c_int]
        hip.hipGetErrorString.restype = ctypes.c_char_p
        e = hip.hipGetLastError()
        if e == 0:
            return ""
        return f" [{hip.hipGetErrorName(e).decode()} ({e}): {hip.hipGetErrorString(e).decode()}]"
    except (OSError, AttributeError):
        return ""


class KvdError(RuntimeError):
    def __init__(self, status: int, where: str):
        detail = _hip_error() if status == KVD_ERR_HIP else ""
        super().__init__(f"{where}: {status_str(status)} (status {status}){detail}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_pool_blocks", ctypes.c_int32), ("max_context_len", ctypes.c_int32),
                ("partition_size", ctypes.c_int32), ("partitions_per_wave", ctypes.c_int32),
                ("queries_per_seq", ctypes.c_int32), ("mean_context_len", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


_ATTN_ARGS = [ctypes.POINTER(Dims), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
              ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p,
              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]


def hip_runtimes_mapped() -> list[str]:
    """Files of the HIP runtime (libamdhip64) mapped into this process."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            parts = line.split()
            if len(parts) >= 6 and os.path.basename(parts[5]).startswith("libamdhip64"):
                paths.add(os.path.realpath(parts[5]))
    return sorted(paths)


def load() -> ctypes.CDLL:
    """Load the built library (raises if it is missing).

    torch ships its own HIP runtime.  The library links the system one by soname, so it is
    loaded after torch, whose runtime then satisfies that dependency: one HIP runtime per
    process.  Loaded first, it would bring in the system runtime and torch a second one, and
    the two would not share streams or memory (launches fail, later calls crash)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        try:
            import torch  # noqa: F401  (its HIP runtime must be loaded first)
        except ImportError:
            pass
        lib = ctypes.CDLL(_LIB_PATH)
        runtimes = hip_runtimes_mapped()
        if len(runtimes) > 1:
            raise RuntimeError("two HIP runtimes are loaded in this process (" + ", ".join(runtimes)
                               + "); import torch before anything that loads a HIP runtime")
        lib.kvd_workspace_bytes.argtypes = [ctypes.POINTER(Dims)]
        lib.kvd_workspace_bytes.restype = ctypes.c_size_t
        for name in ("kvd_decode_attn_paged", "kvd_decode_partitions", "kvd_reduce_partitions"):
            f = getattr(lib, name)
            f.argtypes = _ATTN_ARGS
            f.restype = ctypes.c_int
        lib.kvd_decode_attn_paged_noalloc.argtypes = _ATTN_ARGS[:15] + [ctypes.c_void_p]
        lib.kvd_decode_attn_paged_noalloc.restype = ctypes.c_int
        lib.kvd_dequant_gather.argtypes = [ctypes.POINTER(Dims), ctypes.c_int, ctypes.c_int,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_void_p]
        lib.kvd_dequant_gather.restype = ctypes.c_int
        lib.kvd_dequant_operands.argtypes = [ctypes.POINTER(Dims), ctypes.c_int, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                             ctypes.c_void_p]
        lib.kvd_dequant_operands.restype = ctypes.c_int
        lib.kvd_append_kv.argtypes = [ctypes.POINTER(Dims), ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p]
        lib.kvd_append_kv.restype = ctypes.c_int
        lib.kvd_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]
        lib.kvd_read_probe.restype = ctypes.c_int
        lib.kvd_status_str.argtypes = [ctypes.c_int]
        lib.kvd_status_str.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def status_str(status: int) -> str:
    return load().kvd_status_str(status).decode()


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _fmt(fmt) -> int:
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def workspace_bytes(dims: Dims) -> int:
    return int(load().kvd_workspace_bytes(ctypes.byref(dims)))


def _attn(name, dims, q, k_cache, v_cache, block_table, context_lens, fmt, scales, codebook,
          sign_pattern, softmax_scale, window, softcap, out, workspace, stream, alibi_slopes):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = getattr(load(), name)(ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                               _ptr(block_table), _ptr(context_lens), _fmt(fmt), _ptr(scales),
                               _ptr(codebook), _ptr(sign_pattern), float(softmax_scale),
                               _ptr(window), float(softcap), _ptr(alibi_slopes), _ptr(out),
                               _ptr(workspace), ws_bytes, _stream(stream))
    if st != 0:
        raise KvdError(st, name)
    return out


def decode_attn_paged(dims, q, k_cache, v_cache, block_table, context_lens, fmt, scales,
                      codebook, sign_pattern, softmax_scale, window, softcap, out, workspace,
                      stream=None, alibi_slopes=None):
    """Both phases; see kvd_decode_attn_paged in include/kvdecode.h."""
    return _attn("kvd_decode_attn_paged", dims, q, k_cache, v_cache, block_table, context_lens,
                 fmt, scales, codebook, sign_pattern, softmax_scale, window, softcap, out,
                 workspace, stream, alibi_slopes)


NOALLOC_WORKSPACE_BYTES = 128 << 20   # KVD_NOALLOC_WORKSPACE_BYTES


def decode_attn_paged_noalloc(dims, q, k_cache, v_cache, block_table, context_lens, fmt, scales,
                              codebook, sign_pattern, softmax_scale, window, softcap, out,
                              stream=None, alibi_slopes=None):
    """Both phases with the library's own static workspace (no allocation); see
    kvd_decode_attn_paged_noalloc in include/kvdecode.h."""
    name = "kvd_decode_attn_paged_noalloc"
    st = load().kvd_decode_attn_paged_noalloc(
        ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(context_lens), _fmt(fmt), _ptr(scales), _ptr(codebook), _ptr(sign_pattern),
        float(softmax_scale), _ptr(window), float(softcap), _ptr(alibi_slopes), _ptr(out),
        _stream(stream))
    if st != 0:
        raise KvdError(st, name)
    return out


def decode_partitions(dims, q, k_cache, v_cache, block_table, context_lens, fmt, scales,
                      codebook, sign_pattern, softmax_scale, window, softcap, out, workspace,
                      stream=None, alibi_slopes=None):
    """Phase 1 (partition kernel) only."""
    return _attn("kvd_decode_partitions", dims, q, k_cache, v_cache, block_table, context_lens,
                 fmt, scales, codebook, sign_pattern, softmax_scale, window, softcap, out,
                 workspace, stream, alibi_slopes)


def reduce_partitions(dims, q, k_cache, v_cache, block_table, context_lens, fmt, scales,
                      codebook, sign_pattern, softmax_scale, window, softcap, out, workspace,
                      stream=None, alibi_slopes=None):
    """Phase 2 (reduce kernel) only."""
    return _attn("kvd_reduce_partitions", dims, q, k_cache, v_cache, block_table, context_lens,
                 fmt, scales, codebook, sign_pattern, softmax_scale, window, softcap, out,
                 workspace, stream, alibi_slopes)


def dequant_gather(dims, fmt, is_v, cache, scales, codebook, block_table, seq, kv_head,
                   token_begin, n_tokens, out, stream=None):
    """Dequantised values of tokens [token_begin, token_begin + n_tokens) -> out fp32 [n, D]."""
    st = load().kvd_dequant_gather(ctypes.byref(dims), _fmt(fmt), int(bool(is_v)), _ptr(cache),
                                   _ptr(scales), _ptr(codebook), _ptr(block_table), int(seq),
                                   int(kv_head), int(token_begin), int(n_tokens), _ptr(out),
                                   _stream(stream))
    if st != 0:
        raise KvdError(st, "kvd_dequant_gather")
    return out


def dequant_operands(dims, fmt, k_cache, v_cache, scales, codebook, block_table, seq, kv_head,
                     pair_begin, n_pairs, out, stream=None):
    """The partition kernel's matrix-core operands of page pairs [pair_begin, pair_begin +
    n_pairs) of one (sequence, KV head) -> out uint32 [n_pairs][64][head_dim + 16]
    (kvd_dequant_operands)."""
    st = load().kvd_dequant_operands(ctypes.byref(dims), _fmt(fmt), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(scales), _ptr(codebook), _ptr(block_table), int(seq),
                                     int(kv_head), int(pair_begin), int(n_pairs), _ptr(out),
                                     _stream(stream))
    if st != 0:
        raise KvdError(st, "kvd_dequant_operands")
    return out


def read_probe(buf, chunk_ids, chunk_bytes, waves_per_cu, loads_in_flight, sink, stream=None):
    """HBM read probe (kvd_read_probe): read the chunks of the uint8 device tensor `buf` listed
    in the int32 tensor `chunk_ids`."""
    st = load().kvd_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(chunk_ids),
                               chunk_ids.numel(), int(chunk_bytes), int(waves_per_cu),
                               int(loads_in_flight), _ptr(sink), sink.numel() * sink.element_size(),
                               _stream(stream))
    if st != 0:
        raise KvdError(st, "kvd_read_probe")


def append_kv(dims, fmt, k_new, v_new, block_table, positions, n_new, k_cache, v_cache, scales,
              codebook=None, sign_pattern=None, stream=None):
    """Write n_new new tokens per sequence (k_new / v_new fp32 [B][n_new][Hkv][D]) into the
    paged cache in place (kvd_append_kv)."""
    st = load().kvd_append_kv(ctypes.byref(dims), _fmt(fmt), _ptr(k_new), _ptr(v_new),
                              _ptr(block_table), _ptr(positions), int(n_new), _ptr(k_cache),
                              _ptr(v_cache), _ptr(scales), _ptr(codebook), _ptr(sign_pattern),
                              _stream(stream))
    if st != 0:
        raise KvdError(st, "kvd_append_kv")


load()
