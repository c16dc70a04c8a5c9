// probe.hip -- a plain streaming read of device memory: the HBM read rate
// this part reaches in practice with nothing else to do (16-byte
// non-temporal loads, a grid over every CU), the ceiling against which the
// expert kernels' algorithmic rates are read.  Its shape is the fastest of a
// sweep over loads in flight per thread (2 to 32) and workgroups per CU (1 to
// 32) on a 2 GiB buffer: one 256-thread workgroup per CU with eight loads in
// flight per thread (32 KB per CU) reached 7.2-7.3 TB/s; more in flight per
// CU streams slower (eight workgroups with four loads each: 6.0-6.2 TB/s).
#include "internal.h"

namespace coli {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;     // 16-byte loads in flight per thread
constexpr int kProbeBlocksPerCU = 1;

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4 *__restrict__ src, size_t n16,
                                                                   uint32_t *sink) {
    const size_t per_block = static_cast<size_t>(kProbeThreads) * kProbeUnroll;
    const size_t stride = static_cast<size_t>(gridDim.x) * per_block;
    uint32_t acc = 0;
    for (size_t base = static_cast<size_t>(blockIdx.x) * per_block + threadIdx.x; base < n16; base += stride) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const size_t i = base + static_cast<size_t>(u) * kProbeThreads;
            v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // The XOR of every word read, so no load can be dropped: one atomic per wave.
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_xor(sink, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_probe_read(const void *buf, size_t bytes, uint32_t *sink, int n_cu, hipStream_t s) {
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    const size_t per_block = static_cast<size_t>(kProbeThreads) * kProbeUnroll;
    size_t blocks = (n16 + per_block - 1) / per_block;
    const size_t cap = static_cast<size_t>(n_cu > 0 ? n_cu : 1) * kProbeBlocksPerCU;
    if (blocks > cap) blocks = cap;
    launch(probe_read_kernel, static_cast<unsigned>(blocks), kProbeThreads, 0, s,
           static_cast<const u32x4 *>(buf), n16, sink);
    return hipGetLastError();
}

}  // namespace coli
