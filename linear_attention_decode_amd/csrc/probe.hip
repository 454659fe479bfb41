// probe.hip -- HBM streaming probes: the bandwidth ceiling the decode,
// flush and eager kernels are measured against, and a plain copy whose
// hardware byte counters calibrate the traffic counters of the others.
#include "device_common.h"

namespace replay {

constexpr int kProbeBlocks = 2048;

// Read every 16-byte word once; the xor of all words decides a store that
// never happens in practice but keeps every load alive.
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4 *src, size_t n16, float *dst) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        const u32x4 b = __builtin_nontemporal_load(src + i + stride);
        const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == 0x9E3779B9u) dst[blockIdx.x] = (float)x;
}

__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4 *src, u32x4 *dst, size_t n16) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

hipError_t launch_probe(int mode, const void *src, void *dst, size_t bytes, hipStream_t s) {
    const size_t n16 = bytes / 16;
    if (mode == 0) {
        probe_read_kernel<<<kProbeBlocks, 256, 0, s>>>(static_cast<const u32x4 *>(src), n16,
                                                      static_cast<float *>(dst));
    } else {
        probe_copy_kernel<<<kProbeBlocks, 256, 0, s>>>(static_cast<const u32x4 *>(src),
                                                      static_cast<u32x4 *>(dst), n16);
    }
    return hipGetLastError();
}

}  // namespace replay
