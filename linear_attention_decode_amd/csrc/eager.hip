// eager.hip -- the eager per-token baseline for gfx950.
//
//     S_out = a S_in + dt v k^T,   y = S_out q
// (page "ReplaySSM: Cachear Inputs, No Estado", section "La solucion",
// eq. "Forma resumen"; section "El problema": every token reads and writes
// the whole state).  It is the comparison point of the buffered path and is
// built with the same streaming tiling: one workgroup per (sequence, head),
// 16-byte coalesced chunks, transposed row reduction for y.
#include "device_common.h"

namespace replay {

template <int P, int N>
struct EagerShape {
    static constexpr int VEC = 4;
    static constexpr int CHUNKS = P * N / VEC;
    static constexpr int NT = CHUNKS < 256 ? CHUNKS : 256;
    static constexpr int ITER = CHUNKS / NT;
    static constexpr int LPR = N / VEC;
    static constexpr int RPI = NT / LPR;
    static_assert(CHUNKS % NT == 0 && NT % 64 == 0, "bad tiling");
};

template <int P, int N, bool IOB>
__global__ __launch_bounds__((EagerShape<P, N>::NT)) void eager_kernel(EagerArgs args) {
    using Sh = EagerShape<P, N>;
    constexpr int VEC = Sh::VEC, NT = Sh::NT, ITER = Sh::ITER, LPR = Sh::LPR, RPI = Sh::RPI;
    using RR = RowReduce<ITER, LPR>;

    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int b = lid / args.H, h = lid % args.H;
    const int g = (h * args.G) / args.H;
    const int tid = threadIdx.x, lane = tid & 63;
    const size_t bh = (size_t)b * args.H + h;
    const size_t tile = bh * (size_t)(P * N);

    Chunk<ST_F32, VEC> ch[ITER];
#pragma unroll
    for (int i = 0; i < ITER; ++i) ch[i].load(args.S_in, tile + (size_t)(i * NT + tid) * VEC);

    const float at = args.a[bh], dtt = args.dt[bh];
    const int col0 = (tid % LPR) * VEC;
    const size_t gq = ((size_t)b * args.G + g) * N + col0;
    float kk[VEC], qq[VEC];
    load_io4<IOB>(args.k, gq, kk);
    load_io4<IOB>(args.q, gq, qq);
    float u[ITER];
#pragma unroll
    for (int i = 0; i < ITER; ++i)
        u[i] = dtt * load_io1<IOB>(args.v, bh * P + i * RPI + tid / LPR);

    float part[ITER][1];
#pragma unroll
    for (int i = 0; i < ITER; ++i) {
        float x[VEC];
        ch[i].widen(x, 1.0f);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            x[e] = fmaf(u[i], kk[e], at * x[e]);
            acc = fmaf(x[e], qq[e], acc);
        }
        f32x4 o = {x[0], x[1], x[2], x[3]};
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4 *>(args.S_out + tile + (size_t)(i * NT + tid) * VEC));
        part[i][0] = acc;
    }
    RR::template run<1>(part, lane);
    if (RR::writer(lane)) {
        const int hi = RR::halving_index(lane);
#pragma unroll
        for (int e = 0; e < RR::FINAL; ++e) {
            const int row = (e + RR::FINAL * hi) * RPI + tid / LPR;
            args.y[bh * P + row] = part[e][0];
        }
    }
}

template <int P, int N>
static hipError_t launch_one(const EagerArgs &a, hipStream_t s) {
    const unsigned blocks = (unsigned)((size_t)a.B * a.H);
    if (a.io_bf16)
        eager_kernel<P, N, true><<<blocks, EagerShape<P, N>::NT, 0, s>>>(a);
    else
        eager_kernel<P, N, false><<<blocks, EagerShape<P, N>::NT, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_eager(int P, int N, const EagerArgs &a, hipStream_t s) {
    if (P == 16 && N == 16) return launch_one<16, 16>(a, s);
    if (P == 64 && N == 64) return launch_one<64, 64>(a, s);
    if (P == 64 && N == 128) return launch_one<64, 128>(a, s);
    if (P == 128 && N == 128) return launch_one<128, 128>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace replay
