// probe.hip -- HBM streaming probes: the bandwidth ceiling the decode,
// flush and eager kernels are measured against, and a plain copy whose
// hardware byte counters calibrate the traffic counters of the others.
#include "device_common.h"

namespace replay {

// One 32 KiB tile per workgroup: 256 lanes x 8 words of 16 bytes, every load
// issued before any is used, non-temporal (the access pattern of the
// decode kernels' checkpoint stream).
constexpr int kProbeWords = 256 * 8;

// Read every 16-byte word once; the xor of all words decides a store that
// never happens in practice but keeps every load alive.
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4 *src, size_t n16, float *dst) {
    const size_t base = (size_t)blockIdx.x * kProbeWords + threadIdx.x;
    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const size_t k = base + (size_t)i * 256;
        v[i] = k < n16 ? __builtin_nontemporal_load(src + k) : u32x4{0u, 0u, 0u, 0u};
    }
    u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) acc ^= v[i];
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == 0x9E3779B9u) dst[blockIdx.x] = (float)x;
}

__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4 *src, u32x4 *dst, size_t n16) {
    const size_t base = (size_t)blockIdx.x * kProbeWords + threadIdx.x;
    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const size_t k = base + (size_t)i * 256;
        if (k < n16) v[i] = __builtin_nontemporal_load(src + k);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const size_t k = base + (size_t)i * 256;
        if (k < n16) __builtin_nontemporal_store(v[i], dst + k);
    }
}

hipError_t launch_probe(int mode, const void *src, void *dst, size_t bytes, hipStream_t s) {
    const size_t n16 = bytes / 16;
    const size_t grid = (n16 + kProbeWords - 1) / kProbeWords;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffffu) return hipErrorInvalidValue;
    if (mode == 0) {
        probe_read_kernel<<<(unsigned)grid, 256, 0, s>>>(static_cast<const u32x4 *>(src), n16,
                                                        static_cast<float *>(dst));
    } else {
        probe_copy_kernel<<<(unsigned)grid, 256, 0, s>>>(static_cast<const u32x4 *>(src),
                                                        static_cast<u32x4 *>(dst), n16);
    }
    return hipGetLastError();
}

}  // namespace replay
