// step_copy.hip -- append + output-only decode in one launch, reading a
// low-precision checkpoint copy (bf16, e4m3 or MX FP4) with bf16 io.  The
// library routes e4m3 and FP4 copies here; with a bf16 copy the append and
// decode kernels in turn measured faster.
//
// For every (sequence, head): this step's token goes into the ring and
//     y = abar_t (S q_t) + sum_{j<=t} s_{j,t} v_j (k_j . q_t)
// is produced from the copy S (page "ReplaySSM: Cachear Inputs, No Estado",
// section "Los dos caminos", eq. "Ruta solo salida"; page "ReplaySSM: Cache
// SSM Inputs, Not State", Abstract: a low-precision copy serves the outputs
// while the higher-precision checkpoint takes the updates).  The fold stays
// with the flush kernel, which runs after this one.
//
// The workgroup is the decode kernel's several-head workgroup for the copy
// (the heads' tiles stream as one taller tile, bf16-pair dot products) with
// the fused step's ring wavefronts, one per head and 16-entry block: each
// takes this step's token from the inputs and arrives at its group's
// counter.  A writer workgroup per sequence, after all of them in the grid,
// copies the token into ring slot pos mod L and arrives too; the last
// arrival moves pos.  Where the stacked tiles stream with one wavefront per
// head (L <= 16, P <= 64), step_copy_fused_kernel gives each streaming
// wavefront its head's ring work instead.
// Outputs equal those of the append and decode kernels run in turn, bit for
// bit.
#include "step_common.h"
#include "decode_impl.h"

namespace replay {

template <int P, int N, int ST, int LM, int HPW>
struct StepCopyLaunch {
    using Sh = DecodeShape<P * HPW, N, ST, 1, false>;
    static constexpr int NR = LM / 16;                 // ring wavefronts per head
    static constexpr int NT = Sh::NTS + 64 * NR * HPW;
};

template <int P, int N, int ST, int LM, int HPW>
__global__ __launch_bounds__((StepCopyLaunch<P, N, ST, LM, HPW>::NT)) void step_copy_kernel(StepArgs args) {
    using SL = StepCopyLaunch<P, N, ST, LM, HPW>;
    using Sh = typename SL::Sh;
    constexpr int VEC = Sh::VEC, NTS = Sh::NTS, ITER = Sh::ITER, LPR = Sh::LPR, RPI = Sh::RPI;
    constexpr int NR = SL::NR, PT = P * HPW;
    using RR = RowReduce<ITER, LPR>;

    __shared__ float s_r[NR][HPW][P];
    __shared__ float s_abar[HPW];
    __shared__ __align__(16) float s_sw[HPW][LM];
    __shared__ int s_route;   // 0 output, 2 error (sequence left unchanged)

    const int H = args.H, G = args.G, L = args.L;
    const int HW = H / HPW;
    const int ncomp = args.B * HW;   // compute workgroups; one writer per sequence follows
    if ((int)blockIdx.x >= ncomp) {
        step_token_writer<P, N, true, false>(args, (int)blockIdx.x - ncomp, threadIdx.x, blockDim.x);
        return;
    }
    const int lid = xcd_remap(blockIdx.x, ncomp);
    const int b = lid / HW, h0 = (lid % HW) * HPW;
    const int g = (h0 * G) / H;   // the HPW heads share this group
    const int tid = threadIdx.x, lane = tid & 63;
    // wave-uniform role: scalar branches
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool streamer = wave < NTS / 64;
    const int rw = wave - NTS / 64;
    const size_t bh0 = (size_t)b * H + h0;
    const size_t tile = bh0 * (size_t)(P * N);

    if (streamer) {
        // the copy's tile chunks first, then this step's (group-shared) query as bf16 pairs
        Chunk<ST, VEC> ch[ITER];
#pragma unroll
        for (int i = 0; i < ITER; ++i) {
            if constexpr (ST == ST_FP4)
                ch[i].load_mx(args.copy, args.copy_scale, tile + (size_t)(i * NTS + tid) * VEC);
            else
                ch[i].load(args.copy, tile + (size_t)(i * NTS + tid) * VEC);
        }
        const int col0 = (tid % LPR) * VEC;
        constexpr int QW = VEC / 2;
        uint32_t qw[QW];
        const uint32_t *row = reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(args.q) +
                                                                  ((size_t)b * G + g) * N + col0);
        if constexpr (QW % 4 == 0) {
#pragma unroll
            for (int e = 0; e < QW / 4; ++e) {
                const uint4 u = reinterpret_cast<const uint4 *>(row)[e];
                qw[4 * e] = u.x; qw[4 * e + 1] = u.y; qw[4 * e + 2] = u.z; qw[4 * e + 3] = u.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < QW; ++e) qw[e] = row[e];
        }
        float part[ITER][1];
#pragma unroll
        for (int i = 0; i < ITER; ++i) {
            float acc = ch[i].dot_bf16(qw);
            if constexpr (ST == ST_FP4) acc = ldexpf(acc, ch[i].se);   // the block's scale, exact
            part[i][0] = acc;
        }
        RR::template run<1>(part, lane);
        // LDS-only barrier: the ring writes and arrival atomics finish in the background
        lds_barrier();
        if (s_route != 0) {
            for (int i = tid; i < PT; i += NTS) args.y[bh0 * P + i] = __builtin_nanf("");
            return;
        }
        if (RR::writer(lane)) {
            const int hi = RR::halving_index(lane);
#pragma unroll
            for (int e = 0; e < RR::FINAL; ++e) {
                const int row_ = (e + RR::FINAL * hi) * RPI + tid / LPR;   // of the HPW stacked tiles
                const int hl = HPW == 1 ? 0 : row_ / P, p = HPW == 1 ? row_ : row_ % P;
                const float sc = (ST == ST_FP8) ? static_cast<const float *>(args.copy_scale)[bh0 + hl] : 1.0f;
                float rt = s_r[0][hl][p];
                if constexpr (NR == 2) rt += s_r[1][hl][p];   // block 0 + block 1
                args.y[bh0 * P + row_] = s_abar[hl] * (sc * part[e][0]) + rt;
            }
        }
    } else {
        const int hl = rw / NR, blk = rw % NR;   // head h0 + hl, 16-entry block blk
        const int h = h0 + hl;
        const size_t bh = bh0 + hl;
        const int base = args.base[b];
        const int pos = args.pos[b];
        const int cold = pos - base;
        const bool bad = cold + 1 > L || pos == 2147483647;
        if (rw == 0 && lane == 0) {
            s_route = bad ? 2 : 0;
            if (bad) raise_seq_error(args.err, b, cold + 1 > L ? REPLAY_SEQERR_RING_OVERFLOW : REPLAY_SEQERR_POS_OVERFLOW);
        }
        int prev = -1;
        if (!bad) {
            StepRingMx<P, N, LM> sr;
            sr.load(args, lane, blk, b, g, h, bh, base, cold);
            prev = sr.finish(args, lane, b, g, cold, false, &s_r[blk][hl], &s_abar[hl],
                             static_cast<float (*)[LM + 1]>(nullptr), static_cast<float (*)[N]>(nullptr), &s_sw[hl]);
        }
        lds_barrier();
        if (lane == 0 && prev == NR * (H / G) - 1) {
            // last ring wavefront of the group: the group arrives at the
            // sequence's counter
            atomicExch(args.sync + ((size_t)b * (G + 1) + g) * kSyncStride, 0);
            step_seq_arrive(args, b, pos, false);
        }
    }
}

// The same step with no wavefront set aside for the ring (L <= 16, P <= 64,
// and copy tiles that stream with one wavefront per head): every wavefront
// reads the pointer, issues its share of the stacked tiles, then its head's
// ring loads, and forms the row dot products while those fly.  A workgroup
// is half as many wavefronts, so a CU holds more of them (register-bound:
// 5 to 8 per SIMD instead of 4 workgroups of 8 wavefronts).  The streaming
// and ring arithmetic is the kernel's above, value for value.
template <int P, int N, int ST, int HPW>
struct StepCopyFused {
    using Sh = DecodeShape<P * HPW, N, ST, 1, false>;
    static constexpr int NT = Sh::NTS;
    static constexpr bool fits = HPW > 1 && P <= 64 && Sh::NTS == 64 * HPW;
};

template <int P, int N, int ST, int HPW>
__global__ __launch_bounds__(64 * HPW) __attribute__((amdgpu_waves_per_eu(5))) void step_copy_fused_kernel(StepArgs args) {
    using Sh = typename StepCopyFused<P, N, ST, HPW>::Sh;
    constexpr int LM = 16;
    constexpr int VEC = Sh::VEC, NTS = Sh::NTS, ITER = Sh::ITER, LPR = Sh::LPR, RPI = Sh::RPI;
    static_assert(NTS == 64 * HPW, "one wavefront per head");
    using RR = RowReduce<ITER, LPR>;

    __shared__ float s_r[HPW][P];
    __shared__ float s_abar[HPW];
    __shared__ __align__(16) float s_sw[HPW][LM];

    const int H = args.H, G = args.G, L = args.L;
    const int HW = H / HPW;
    const int ncomp = args.B * HW;   // compute workgroups; one writer per sequence follows
    if ((int)blockIdx.x >= ncomp) {
        step_token_writer<P, N, true, false>(args, (int)blockIdx.x - ncomp, threadIdx.x, blockDim.x);
        return;
    }
    const int lid = xcd_remap(blockIdx.x, ncomp);
    const int b = lid / HW, h0 = (lid % HW) * HPW;
    const int g = (h0 * G) / H;   // the HPW heads share this group
    const int tid = threadIdx.x, lane = tid & 63;
    const int hl = __builtin_amdgcn_readfirstlane(tid >> 6);   // this wavefront's ring head
    const size_t bh0 = (size_t)b * H + h0;
    const size_t tile = bh0 * (size_t)(P * N);

    // the pointer through the scalar cache (b is uniform; nothing in this
    // launch writes pos or base before every wavefront of the sequence has
    // read them)
    using cint = const __attribute__((address_space(4))) int;
    const int base = *((cint *)args.base + b);
    const int pos = *((cint *)args.pos + b);
    // this step's token (the group's query row, one word a lane, serves the
    // ring and the tile's dot products), then the copy's tile chunks
    StepRingMx<P, N, LM> sr;
    sr.load_token(args, lane, b, g, bh0 + hl);
    Chunk<ST, VEC> ch[ITER];
#pragma unroll
    for (int i = 0; i < ITER; ++i) {
        if constexpr (ST == ST_FP4)
            ch[i].load_codes(args.copy, tile + (size_t)(i * NTS + tid) * VEC);
        else
            ch[i].load(args.copy, tile + (size_t)(i * NTS + tid) * VEC);
    }
    // FP4: the wavefront's ITER runs of 64 block scales (one byte per lane and
    // chunk), one word a lane
    uint32_t sword = 0;
    if constexpr (ST == ST_FP4) {
        static_assert(VEC == 32 && ITER <= 4, "one scale byte per lane and chunk, one word per lane in all");
        const int seg = lane >> 4;
        const size_t sb = tile / 32 + (size_t)(seg < ITER ? seg : 0) * NTS + (size_t)(tid & ~63) + 4 * (lane & 15);
        sword = *reinterpret_cast<const uint32_t *>(static_cast<const uint8_t *>(args.copy_scale) + sb);
    }
    const int cold = pos - base;
    const bool bad = cold + 1 > L || pos == 2147483647;
    if (!bad) sr.load_ring(args, lane, 0, b, g, bh0 + hl, base, cold);

    // the query as bf16 pairs at this lane's columns: words (tid % LPR) QW .. + QW - 1 of the row
    constexpr int QW = VEC / 2;
    static_assert(RowWords<N, true>::WPL == 1, "one word of the row per lane");
    uint32_t qw[QW];
#pragma unroll
    for (int e = 0; e < QW; ++e) qw[e] = (uint32_t)__shfl((int)sr.qrow.w[0], (tid % LPR) * QW + e);
    if constexpr (ST == ST_FP4) {
#pragma unroll
        for (int i = 0; i < ITER; ++i)
            ch[i].se = (int)((((uint32_t)__shfl((int)sword, 16 * i + (lane >> 2))) >> (8 * (lane & 3))) & 0xffu) - 127;
    }

    float part[ITER][1];
#pragma unroll
    for (int i = 0; i < ITER; ++i) {
        float acc = ch[i].dot_bf16(qw);
        if constexpr (ST == ST_FP4) acc = ldexpf(acc, ch[i].se);   // the block's scale, exact
        part[i][0] = acc;
    }
    RR::template run<1>(part, lane);

    if (bad) {   // sequence left unchanged
        if (tid == 0) raise_seq_error(args.err, b, cold + 1 > L ? REPLAY_SEQERR_RING_OVERFLOW : REPLAY_SEQERR_POS_OVERFLOW);
        for (int i = tid; i < P * HPW; i += NTS) args.y[bh0 * P + i] = __builtin_nanf("");
        return;
    }
    const int prev = sr.finish(args, lane, b, g, cold, false, &s_r[hl], &s_abar[hl],
                               static_cast<float (*)[LM + 1]>(nullptr), static_cast<float (*)[N]>(nullptr), &s_sw[hl]);
    // LDS-only barrier: the arrival atomics finish in the background
    lds_barrier();
    if (RR::writer(lane)) {
        const int hi = RR::halving_index(lane);
#pragma unroll
        for (int e = 0; e < RR::FINAL; ++e) {
            const int row_ = (e + RR::FINAL * hi) * RPI + tid / LPR;   // of the HPW stacked tiles
            const int hr = row_ / P, p = row_ % P;
            const float sc = (ST == ST_FP8) ? static_cast<const float *>(args.copy_scale)[bh0 + hr] : 1.0f;
            args.y[bh0 * P + row_] = s_abar[hr] * (sc * part[e][0]) + s_r[hr][p];
        }
    }
    if (lane == 0 && prev == H / G - 1) {
        // last wavefront of the group: the group arrives at the sequence's counter
        atomicExch(args.sync + ((size_t)b * (G + 1) + g) * kSyncStride, 0);
        step_seq_arrive(args, b, pos, false);
    }
}

template <int P, int N, int ST, int LM>
static hipError_t launch_sc_lm(const StepArgs &a, hipStream_t s) {
    constexpr int HPW = heads_per_wg<ST, 1>();
    if constexpr (LM == 16 && StepCopyFused<P, N, ST, HPW>::fits) {
        if ((a.H / a.G) % HPW == 0) {
            const unsigned blocks = (unsigned)((size_t)a.B * a.H / HPW + a.B);
            step_copy_fused_kernel<P, N, ST, HPW><<<blocks, StepCopyFused<P, N, ST, HPW>::NT, 0, s>>>(a);
            return hipGetLastError();
        }
    }
    if (HPW > 1 && (a.H / a.G) % HPW == 0) {
        const unsigned blocks = (unsigned)((size_t)a.B * a.H / HPW + a.B);
        step_copy_kernel<P, N, ST, LM, HPW><<<blocks, StepCopyLaunch<P, N, ST, LM, HPW>::NT, 0, s>>>(a);
    } else {
        const unsigned blocks = (unsigned)((size_t)a.B * a.H + a.B);
        step_copy_kernel<P, N, ST, LM, 1><<<blocks, StepCopyLaunch<P, N, ST, LM, 1>::NT, 0, s>>>(a);
    }
    return hipGetLastError();
}

template <int P, int N, int ST>
static hipError_t launch_sc_st(const StepArgs &a, hipStream_t s) {
    if (a.L <= 16) return launch_sc_lm<P, N, ST, 16>(a, s);
    return launch_sc_lm<P, N, ST, kMaxRing>(a, s);
}

template <int P, int N>
static hipError_t launch_sc_pn(const StepArgs &a, hipStream_t s) {
    switch (a.copy_st) {
        case ST_BF16: return launch_sc_st<P, N, ST_BF16>(a, s);
        case ST_FP8: return launch_sc_st<P, N, ST_FP8>(a, s);
        case ST_FP4: return launch_sc_st<P, N, ST_FP4>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_step_copy(int P, int N, const StepArgs &a, hipStream_t s) {
    if (!a.io_bf16) return hipErrorInvalidValue;
    if (P == 16 && N == 16) return launch_sc_pn<16, 16>(a, s);
    if (P == 64 && N == 64) return launch_sc_pn<64, 64>(a, s);
    if (P == 64 && N == 128) return launch_sc_pn<64, 128>(a, s);
    if (P == 128 && N == 128) return launch_sc_pn<128, 128>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace replay
