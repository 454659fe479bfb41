// ring.hip -- ring-buffer pointer operations and small utility kernels.
//
// append: tokens go into the ring slot of their absolute index modulo L
// (page "ReplaySSM: Cachear Inputs, No Estado", "Decodificacion estandar":
// recent inputs are kept in a buffer; page "The SSM Layer Nobody Made Fast
// (Until Now): ReplaySSM Explained", key technical takeaways: a ring of the
// L most recent inputs).  rollback: the pointer moves back over rejected
// tokens (same pages, "Rollback" / O(1) pointer decrement).  Both check the
// ring bounds per sequence on the device and set that sequence's error bit
// instead of acting.
#include "device_common.h"

namespace replay {

// kAppendSlices workgroups per sequence, each copying the tokens of its
// share of the heads (v, dt, a) and of the groups (q, k); the last slice to
// arrive at the sequence's counter advances the pointer.  A slice arrives
// only after a workgroup barrier, so every wavefront of every slice has read
// the pointer before any slice can move it.
constexpr int kAppendSlices = 8;

__global__ __launch_bounds__(256) void append_kernel(RingView r, void *ring_q, void *ring_k,
                                                     void *ring_v, float *ring_dt, float *ring_a,
                                                     int32_t *pos, int32_t *sync, int32_t W, const void *q,
                                                     const void *k, const void *v, const float *dt,
                                                     const float *a, int32_t P, int32_t N) {
    const int b = blockIdx.x, sl = blockIdx.y;
    const int tid = threadIdx.x, nt = blockDim.x;
    const int H = r.H, G = r.G, L = r.L;
    const int p0 = pos[b];
    const int count = p0 - r.base[b];
    if (count + W > L) {
        if (sl == 0 && tid == 0) raise_seq_error(r.err, b, REPLAY_SEQERR_RING_OVERFLOW);
        return;
    }
    if ((long long)p0 + W > 2147483647LL) {
        if (sl == 0 && tid == 0) raise_seq_error(r.err, b, REPLAY_SEQERR_POS_OVERFLOW);
        return;
    }
    const int esz = r.io_bf16 ? 2 : 4;
    const int h0 = sl * H / kAppendSlices, h1 = (sl + 1) * H / kAppendSlices;
    const int g0 = sl * G / kAppendSlices, g1 = (sl + 1) * G / kAppendSlices;

    // v rows of heads h0..h1-1: [B][W][H][P] -> [B][H][L][P]; 16-byte pieces
    {
        const int vec_per_row = P * esz / 16;
        const int nh = h1 - h0;
        const int total = W * nh * vec_per_row;
        const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const char *>(v) + (size_t)b * W * H * P * esz);
        for (int i = tid; i < total; i += nt) {
            const int row = i / vec_per_row, c = i % vec_per_row;
            const int t = row / nh, h = h0 + row % nh;
            const int slot = (p0 + t) % L;
            uint4 *dst = reinterpret_cast<uint4 *>(static_cast<char *>(ring_v) +
                                                   (((size_t)b * H + h) * L + slot) * P * esz);
            dst[c] = src[((size_t)t * H + h) * vec_per_row + c];
        }
    }
    // q, k rows of groups g0..g1-1: [B][W][G][N] -> [B][G][L][N]
    {
        const int vec_per_row = N * esz / 16;
        const int ng = g1 - g0;
        const int total = W * ng * vec_per_row;
        const size_t in_off = (size_t)b * W * G * N * esz;
        const uint4 *sq = reinterpret_cast<const uint4 *>(static_cast<const char *>(q) + in_off);
        const uint4 *sk = reinterpret_cast<const uint4 *>(static_cast<const char *>(k) + in_off);
        for (int i = tid; i < total; i += nt) {
            const int row = i / vec_per_row, c = i % vec_per_row;
            const int t = row / ng, gg = g0 + row % ng;
            const int slot = (p0 + t) % L;
            const size_t out_off = (((size_t)b * G + gg) * L + slot) * N * esz;
            const size_t in_row = ((size_t)t * G + gg) * vec_per_row + c;
            reinterpret_cast<uint4 *>(static_cast<char *>(ring_q) + out_off)[c] = sq[in_row];
            reinterpret_cast<uint4 *>(static_cast<char *>(ring_k) + out_off)[c] = sk[in_row];
        }
    }
    // dt, a of heads h0..h1-1: [B][W][H] -> [B][L][H]
    {
        const int nh = h1 - h0;
        for (int i = tid; i < W * nh; i += nt) {
            const int t = i / nh, h = h0 + i % nh;
            const int slot = (p0 + t) % L;
            const size_t o = dta_index(b, (size_t)b * H + h, H, L, slot);
            ring_dt[o] = dt[((size_t)b * W + t) * H + h];
            ring_a[o] = a[((size_t)b * W + t) * H + h];
        }
    }
    // every wavefront of this slice has read pos[b] (and its overflow checks
    // agreed: they all read the same value) before the slice arrives
    __syncthreads();
    if (tid == 0) {
        int32_t *cnt = sync + ((size_t)b * (G + 1) + G) * kSyncStride;
        if (atomicAdd(cnt, 1) == kAppendSlices - 1) {
            atomicExch(cnt, 0);
            pos[b] = p0 + W;
        }
    }
}

__global__ void rollback_kernel(const int32_t *base, int32_t *pos, const int32_t *n_reject,
                                int32_t *err, int32_t B) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const int r = n_reject[b];
    const int p = pos[b];
    if (r < 0 || r > p - base[b]) {
        raise_seq_error(err, b, REPLAY_SEQERR_ROLLBACK_RANGE);
        return;
    }
    pos[b] = p - r;
}

__global__ void fill_u32_kernel(uint32_t *dst, uint32_t value, size_t count) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (size_t)gridDim.x * blockDim.x)
        dst[i] = value;
}

// s[b] <- snaps[n_accept[b] - 1][b] for 1 <= n_accept[b] <= W
__global__ void eager_select_kernel(const float *snaps, int32_t W, const int32_t *n_accept, float *s,
                                    int32_t B, size_t per_seq) {
    const int b = blockIdx.y;
    const int c = n_accept[b];
    if (c < 1 || c > W) return;
    const f32x4 *src = reinterpret_cast<const f32x4 *>(snaps + ((size_t)(c - 1) * B + b) * per_seq);
    f32x4 *dst = reinterpret_cast<f32x4 *>(s + (size_t)b * per_seq);
    const size_t n4 = per_seq / 4;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

hipError_t launch_append(int P, int N, const RingView &r, void *ring_q, void *ring_k, void *ring_v,
                         float *ring_dt, float *ring_a, int32_t *pos, int32_t *sync, int32_t W, const void *q,
                         const void *k, const void *v, const float *dt, const float *a, hipStream_t s) {
    append_kernel<<<dim3(r.B, kAppendSlices), 256, 0, s>>>(r, ring_q, ring_k, ring_v, ring_dt, ring_a, pos, sync,
                                                           W, q, k, v, dt, a, P, N);
    return hipGetLastError();
}

hipError_t launch_rollback(const RingView &r, int32_t *pos, const int32_t *n_reject, hipStream_t s) {
    rollback_kernel<<<(r.B + 255) / 256, 256, 0, s>>>(r.base, pos, n_reject, r.err, r.B);
    return hipGetLastError();
}

hipError_t launch_fill_u32(void *dst, uint32_t value, size_t count, hipStream_t s) {
    if (count == 0) return hipSuccess;
    size_t blocks = (count + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    fill_u32_kernel<<<(unsigned)blocks, 256, 0, s>>>(static_cast<uint32_t *>(dst), value, count);
    return hipGetLastError();
}

hipError_t launch_eager_select(const float *snaps, int32_t W, const int32_t *n_accept, float *s,
                               int32_t B, size_t per_seq, hipStream_t st) {
    dim3 grid(64, B);
    eager_select_kernel<<<grid, 256, 0, st>>>(snaps, W, n_accept, s, B, per_seq);
    return hipGetLastError();
}

}  // namespace replay
