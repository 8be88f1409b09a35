// HBM read probe (measurement export): how fast the chip streams memory when its waves read
// chunks of a buffer in a given order -- consecutive (a plain read stream) or at random chunk
// indices (the access pattern of a paged cache, whose pages sit at random places in the pool).
// It gives the decode kernels' roofline its practical ceiling: the bytes a random-page read can
// deliver per second with the same chunk sizes and in-flight bytes per wave.
#include <stdint.h>

#include "kvd_internal.h"

namespace kvd {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Waves read the flat list of 1 KB pieces (chunk ids[c], piece k), U consecutive pieces per wave
// turn (U KB in flight per wave: all U loads are issued before any is used), then the next
// turn nwaves * U pieces further on.  The data is folded into one word per lane and stored, so
// no load can be dropped.  Chunk ids outside the buffer read chunk 0 instead.
template <int U>
__global__ __launch_bounds__(256) void read_probe_kernel(const ProbeParams p) {
    const int lane = threadIdx.x & 63;
    // wave-uniform, so the chunk ids come in with scalar loads
    const int64_t wave = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    const int sh = p.log2_pieces;                       // 1 KB pieces per chunk: 1 << sh
    const int64_t items = p.n << sh;
    const int64_t chunks_in_buf = p.buf_bytes >> (sh + 10);
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t base = wave * U; base < items; base += nwaves * U) {
        int64_t addr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {   // chunk ids first, so their loads overlap
            const int64_t it = base + u < items ? base + u : items - 1;
            int64_t id = p.ids[it >> sh];
            if (id < 0 || id >= chunks_in_buf) id = 0;
            addr[u] = ((id << sh) + (it & ((1 << sh) - 1))) * 1024 + lane * 16;
        }
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const u32x4*>(p.buf + addr[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    p.sink[wave * 64 + lane] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

hipError_t launch_read_probe(const ProbeParams& p, int blocks, int loads_in_flight, hipStream_t s) {
    const dim3 grid(blocks), block(256);
    switch (loads_in_flight) {
        case 1: return launch_kernel(read_probe_kernel<1>, grid, block, s, p);
        case 2: return launch_kernel(read_probe_kernel<2>, grid, block, s, p);
        case 4: return launch_kernel(read_probe_kernel<4>, grid, block, s, p);
        case 8: return launch_kernel(read_probe_kernel<8>, grid, block, s, p);
        default: return launch_kernel(read_probe_kernel<16>, grid, block, s, p);
    }
}

}  // namespace kvd
