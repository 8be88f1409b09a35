"""GPU: the HBM read probe reads exactly the chunks it is given.

kvd_read_probe folds every 16-byte piece a wave reads into one word per lane.  A CPU model of
the documented schedule (wave w reads items w*U .. w*U+U-1, then nwaves*U further on; items past
the end repeat the last one; chunk ids outside the buffer read chunk 0) must give the same
words, so the probe's bandwidth figure counts reads of the right bytes.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _model(buf, ids, chunk_bytes, nwaves, U):
    """Expected sink words [nwaves * 64] (uint32)."""
    words = buf.view(np.uint32).reshape(-1, 4)            # 16-byte pieces
    sh = int(np.log2(chunk_bytes // 1024))
    pieces = 1 << sh
    items = len(ids) * pieces
    n_chunks = len(buf) // chunk_bytes
    lanes = np.arange(64)
    out = np.zeros((nwaves, 64), dtype=np.uint32)
    for w in range(nwaves):
        acc = np.zeros((64, 4), dtype=np.uint32)
        for base in range(w * U, items, nwaves * U):
            for u in range(U):
                it = min(base + u, items - 1)
                cid = int(ids[it >> sh])
                if cid < 0 or cid >= n_chunks:
                    cid = 0
                byte0 = ((cid << sh) + (it & (pieces - 1))) * 1024
                acc ^= words[byte0 // 16 + lanes]
        out[w] = acc[:, 0] ^ acc[:, 1] ^ acc[:, 2] ^ acc[:, 3]
    return out.reshape(-1)


@pytest.mark.parametrize("chunk_bytes,lif,n", [(1024, 4, 700), (2048, 8, 257), (4096, 2, 64)])
def test_read_probe_reads_the_listed_chunks(chunk_bytes, lif, n):
    import torch
    import quantized_kv_cache_split_amd as kvd
    rng = np.random.default_rng(chunk_bytes + lif)
    buf = rng.integers(0, 256, size=4 << 20, dtype=np.uint8)
    n_chunks = len(buf) // chunk_bytes
    ids = rng.permutation(n_chunks)[:n].astype(np.int32)
    ids[3] = -7                      # outside the buffer: reads chunk 0
    ids[5] = n_chunks + 11
    wpc = 4
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nwaves = cus * wpc               # blocks of 4 waves: cus * wpc / 4 of them
    sink = torch.zeros(nwaves * 64, dtype=torch.int32, device="cuda:0")
    tbuf = torch.from_numpy(buf).to("cuda:0")
    tids = torch.from_numpy(ids).to("cuda:0")
    kvd.read_probe(tbuf, tids, chunk_bytes, wpc, lif, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    want = _model(buf, ids, chunk_bytes, nwaves, lif)
    assert np.array_equal(got, want)


def test_read_probe_rejects_bad_arguments():
    import torch
    import quantized_kv_cache_split_amd as kvd
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda:0")
    ids = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(1 << 20, dtype=torch.int32, device="cuda:0")
    for cb, wpc, lif in ((1536, 4, 4), (512, 4, 4), (1024, 6, 4), (1024, 4, 3)):
        with pytest.raises(kvd.KvdError):
            kvd.read_probe(buf, ids, cb, wpc, lif, sink)
