"""The C-ABI library loads, exports every declared symbol, and rejects bad arguments on the
host before anything is launched (no GPU needed: these paths make no HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvdecode.h")

kvd = pytest.importorskip("quantized_kv_cache_split_amd")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kvd_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"kvd_decode_attn_paged", "kvd_decode_partitions", "kvd_reduce_partitions",
            "kvd_workspace_bytes", "kvd_dequant_gather", "kvd_status_str"} <= set(names)
    lib = ctypes.CDLL(kvd.library_path())
    for n in names:
        assert hasattr(lib, n), n


def test_one_hip_runtime_per_process():
    """Loading the library leaves exactly one HIP runtime mapped: torch's, when torch is
    installed (the library binds to it instead of loading the system copy beside it)."""
    kvd.load()
    maps = kvd.hip_runtimes_mapped()
    assert len(maps) == 1, maps
    try:
        import torch
    except ImportError:
        return
    assert os.path.dirname(maps[0]) == os.path.realpath(os.path.join(os.path.dirname(torch.__file__), "lib"))


def test_hip_error_detail_uses_the_mapped_runtime():
    """The error detail of a failed launch is read from the HIP runtime already in the process;
    asking for it never maps a second one (with nothing pending it is empty)."""
    kvd.load()
    before = kvd.hip_runtimes_mapped()
    detail = kvd._hip_error()
    assert kvd.hip_runtimes_mapped() == before
    assert isinstance(detail, str)


def dims(**kw):
    base = dict(num_seqs=16, num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=16,
                max_blocks_per_seq=2048, num_pool_blocks=33792, max_context_len=32768,
                partition_size=0)
    base.update(kw)
    return kvd.Dims(**base)


def test_workspace_bytes():
    d = dims()
    rows = 16 * 64 * 64
    assert kvd.workspace_bytes(d) == 2 * rows * 4 + rows * 128 * 4
    assert kvd.workspace_bytes(dims(max_context_len=1000)) == 0       # auto: never splits
    assert kvd.workspace_bytes(dims(partition_size=-1)) == 0
    assert kvd.workspace_bytes(dims(partition_size=128, max_context_len=300, num_seqs=1,
                                    num_q_heads=4, num_kv_heads=1)) == 256 * 2 + 12 * 128 * 4
    assert kvd.workspace_bytes(dims(head_dim=96)) == 0
    assert kvd.workspace_bytes(dims(partition_size=100)) == 0


def test_status_strings():
    assert kvd.status_str(0) == "ok"
    for s in range(-6, 0):
        assert kvd.status_str(s) != "unknown status"


FAKE = 1 << 20   # a 16-byte aligned, never dereferenced address


def call(d=None, fmt=0, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, ctx=FAKE, scales=FAKE, cb=FAKE, sign=FAKE,
             scale=0.1, win=None, cap=0.0, alibi=None, out=FAKE, ws=FAKE, ws_bytes=1 << 40)
    a.update(over)
    lib = kvd.load()
    return lib.kvd_decode_attn_paged(ctypes.byref(d or dims()), a["q"], a["k"], a["v"], a["bt"],
                                     a["ctx"], fmt, a["scales"], a["cb"], a["sign"], a["scale"],
                                     a["win"], a["cap"], a["alibi"], a["out"], a["ws"],
                                     a["ws_bytes"], None)


@pytest.mark.parametrize("field,value", [("num_q_heads", 60), ("num_kv_heads", 0),
                                         ("head_dim", 96), ("block_size", 32),
                                         ("max_context_len", 0), ("max_context_len", 1 << 20),
                                         ("partition_size", 100), ("partitions_per_wave", -1),
                                         ("mean_context_len", -1)])
def test_shape_errors(field, value):
    assert call(dims(**{field: value})) == -2


def test_turbo_needs_d128():
    assert call(dims(head_dim=64), fmt=2) == -2
    assert call(dims(head_dim=64), fmt=4) == -2      # Turbo8 (codebook V)


def test_format_error():
    assert call(fmt=7) == -3
    assert call(fmt=-1) == -3 and call(fmt=-(1 << 31)) == -3   # negative formats too


def test_size_limits():
    # query rows [B][n_q][Hq] past int32, and a split workspace past 2^62 bytes
    assert call(dims(num_seqs=65535, num_q_heads=1 << 16, num_kv_heads=1)) == -2
    big = dims(num_seqs=4096, num_q_heads=1 << 19, num_kv_heads=1, max_blocks_per_seq=1 << 27,
               max_context_len=(1 << 31) - 1, partition_size=16)
    assert kvd.workspace_bytes(big) == 0 and call(big) == -2
    # runs so long that their token indices would pass int32
    assert call(dims(num_seqs=1, max_blocks_per_seq=1 << 27, max_context_len=(1 << 31) - 64,
                     partition_size=1 << 20, partitions_per_wave=1 << 28)) == -2


@pytest.mark.parametrize("arg", ["q", "k", "v", "bt", "ctx", "out"])
def test_null_errors(arg):
    assert call(**{arg: None}) == -1


def test_fp8_and_turbo_need_their_arrays():
    assert call(fmt=1, scales=None) == -1
    assert call(fmt=2, cb=None) == -1
    assert call(fmt=3, sign=None) == -1
    assert call(fmt=4, scales=None) == -1 and call(fmt=4, cb=None) == -1
    assert call(fmt=4, sign=None) == -1
    assert call(fmt=0, scales=None, cb=None, sign=None, ws_bytes=0) == -5


def test_alibi_alignment_and_large_groups():
    assert call(alibi=FAKE + 2) == -4
    # query groups above 16 (here 64 query heads on one KV head) are accepted
    assert kvd.workspace_bytes(dims(num_q_heads=64, num_kv_heads=1)) > 0


def test_alignment_errors():
    assert call(q=FAKE + 2) == -4
    assert call(ws=FAKE + 16) == -4


def test_workspace_errors():
    assert call(ws=None) == -5
    assert call(ws_bytes=100) == -5


def test_bad_scalars():
    assert call(cap=-1.0) == -2
    assert call(scale=float("nan")) == -2


def test_empty_batch_is_ok_without_launching():
    assert call(dims(num_seqs=0)) == 0


def test_gather_arg_errors():
    lib = kvd.load()
    d = dims()
    g = lambda **k: lib.kvd_dequant_gather(ctypes.byref(d), k.get("fmt", 0), 0, FAKE, FAKE, FAKE,
                                           FAKE, k.get("seq", 0), k.get("head", 0),
                                           k.get("t0", 0), k.get("n", 4), FAKE, None)
    assert g(seq=16) == -2 and g(head=8) == -2 and g(t0=-1) == -2 and g(t0=32768, n=1) == -2
    assert g(fmt=9) == -3
    assert g(n=0) == 0


def append_call(d=None, fmt=0, **over):
    a = dict(k=FAKE, v=FAKE, bt=FAKE, pos=FAKE, n=4, kc=FAKE, vc=FAKE, scales=FAKE, cb=FAKE,
             sign=FAKE)
    a.update(over)
    lib = kvd.load()
    return lib.kvd_append_kv(ctypes.byref(d or dims()), fmt, a["k"], a["v"], a["bt"], a["pos"],
                             a["n"], a["kc"], a["vc"], a["scales"], a["cb"], a["sign"], None)


def test_append_arg_errors():
    assert append_call(fmt=5) == -3
    assert append_call(n=-1) == -2
    assert append_call(dims(head_dim=96)) == -2
    for arg in ("k", "v", "bt", "pos", "kc", "vc"):
        assert append_call(**{arg: None}) == -1, arg
    assert append_call(fmt=1, scales=None) == -1
    assert append_call(fmt=2, cb=None) == -1 and append_call(fmt=3, sign=None) == -1
    assert append_call(fmt=4, scales=None) == -1 and append_call(fmt=4, cb=None) == -1
    assert append_call(fmt=0, scales=None, cb=None, sign=None, n=0) == 0    # BF16 needs neither
    assert append_call(fmt=2, scales=None, n=0) == 0     # Turbo4/3 norms live in the chunks
    assert append_call(fmt=3, scales=None, n=0) == 0
    assert append_call(k=FAKE + 4) == -4 and append_call(kc=FAKE + 8) == -4
    assert append_call(n=0) == 0 and append_call(dims(num_seqs=0)) == 0    # nothing launched


def test_build_script_runs_without_the_package():
    """build() must work in a fresh checkout, where the library does not exist yet: the build
    script is loaded by path (importing it through the package would run the package's
    __init__, which refuses to load before the library is built), and its hipcc line targets
    gfx950 with packed fp32 VALU ops switched off."""
    import importlib.util
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    src = open(os.path.join(root, "__graft_entry__.py")).read()
    assert "spec_from_file_location" in src and "from quantized_kv_cache_split_amd.build" not in src
    spec = importlib.util.spec_from_file_location(
        "_kvd_build_test", os.path.join(root, "quantized_kv_cache_split_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    cmd = mod.command("/tmp/unused.so")
    assert "--offload-arch=gfx950" in cmd
    i = cmd.index("-packed-fp32-ops")
    assert cmd[i - 3:i] == ["-Xclang", "-target-feature", "-Xclang"]
    assert all(s in cmd for s in mod.SOURCES)


def test_noalloc_rejects_oversized_workspace_before_any_hip_call():
    """The allocation-free entry point refuses dims whose partition workspace exceeds its
    static array, and bad shapes, on the host (no GPU needed: nothing is looked up or
    launched)."""
    lib = kvd.load()
    na = lambda d, fmt=0: lib.kvd_decode_attn_paged_noalloc(
        ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, fmt, FAKE, FAKE, FAKE, 0.1, None, 0.0,
        None, FAKE, None)
    big = dims(num_seqs=64, max_context_len=65536, max_blocks_per_seq=4096)   # 68M floats of o
    assert kvd.workspace_bytes(big) > kvd.NOALLOC_WORKSPACE_BYTES
    assert na(big) == -5
    assert na(dims(head_dim=96)) == -2
    assert na(dims(), fmt=9) == -3
    assert kvd.NOALLOC_WORKSPACE_BYTES == 128 << 20
    header = open(HEADER).read()
    assert "#define KVD_NOALLOC_WORKSPACE_BYTES ((size_t)128 << 20)" in header
