// verify_wide.hip -- speculative verify of windows of up to 16 drafts on the
// matrix cores, bf16 io (replay_verify takes it from W = kWideFrom on).
//
// The same outputs as the verify kernel of decode_impl.h: for the W newest
// ring entries t_w = count-W+w of every (sequence, head)
//     y_w = abar_{t_w} (S q_{t_w}) + sum_{j<=t_w} s_{j,t_w} v_j (k_j . q_{t_w})
// against one read of the checkpoint (page "ReplaySSM: Cachear Inputs, No
// Estado", section "Paralelismo": every window position reads the same
// checkpoint and buffer, entry j visible to position t when j <= t; eq. "Ruta
// solo salida").  With W queries every state element enters W products; the
// register kernel's per-row partial sums grow with W (past eight they no
// longer fit), and here S Q^T is formed as a matrix product instead:
//   - streaming wavefront i reads rows 16i..16i+15 of the head's tile in
//     128-byte row segments (8 lanes to a cache line) and turns each 16-row
//     chunk into the matrix cores' operand layout (lane (row r, group g): 16
//     bytes of row 16i+r) through its own small LDS buffer;
//   - the W queries go to LDS as rows Q[w][n] (rows w >= W zero);
//   - D = S Q^T for the 16 rows:
//       float32 tiles: v_mfma_f32_16x16x4_f32, four per 16 columns: the t-th
//         takes column n0+4g+t in lane group g (the contraction order is free;
//         this one lets a lane load four consecutive values once);
//       bf16 tiles: v_mfma_f32_16x16x32_bf16, columns n0+8g..+7 in group g;
//       e4m3 tiles: 16 codes a lane cover two such products (columns
//         n0+16g..+7 and n0+16g+8..+15), turned into bf16 pairs (exact);
//       N below 32: the bf16 and e4m3 values are widened and take the float32
//         products;
//   - the ring wavefront(s) form the ring term for the window (ring_mx.h).
// Output D[p][w] sits in lane (4-row group, column w), register r -> row
// 16i + 4g + r, so each lane writes four consecutive outputs of one query.
#include <type_traits>

#include "decode_impl.h"

namespace replay {

constexpr int kWide = 16;   // columns of D (queries), the MFMA tile width

template <int ST, int N>
constexpr bool wide_bf16_path() { return ST != ST_F32 && N % 32 == 0; }

template <int P, int N, int ST, int LM>
struct WideShape {
    static constexpr bool BF = wide_bf16_path<ST, N>();
    static constexpr int NTS = (P / 16) * 64;                      // one wavefront per 16 rows
    static constexpr int ESZ = ST == ST_F32 ? 4 : (ST == ST_BF16 ? 2 : 1);
    static constexpr int CVEC = BF ? 16 / ESZ : 4;                 // elements a lane loads per step
    static constexpr int STEPS = N / (4 * CVEC);                   // loads per lane (4 lane groups)
    static constexpr int TS = BF ? N + 8 : N + 4;                  // LDS row stride of Q, in elements
    static constexpr int NR = LM / 16;
    static constexpr int NT = NTS + 64 * NR;
    // Coalesced staging (16-byte lane steps, rows of whole 128-byte lines):
    // the tile is read in 128-byte row segments, 8 lanes to a line, and each
    // wavefront turns its 16 x 128-byte chunks into the operand layout
    // through its own LDS buffer.  Loading the operand layout directly makes
    // every load instruction touch 16 half lines, twice the cache requests.
    static constexpr int RB = N * ESZ;   // bytes of a tile row
    static constexpr bool COAL = (ST == ST_F32 || BF) && RB % 128 == 0;
    static constexpr int TROW = 36;      // staging row stride in words (128 bytes + 16 of padding)
    static_assert(!COAL || STEPS == 2 * (RB / 128), "two load steps per 128-byte chunk");
    static_assert(P % 16 == 0 && N % 16 == 0 && N % (4 * CVEC) == 0, "tile shape");
};

// The ring part for a window of W <= 16 positions, operands from the ring
// (as ring_wave_mx of the decode kernel, with the window size at run time).
template <int P, int N, int LM>
__device__ __forceinline__ void wide_ring_wave(const RingView &r, int lane, int j0, int b, int g, size_t bh,
                                               int base, int count, int W, float (*s_r)[P], float *s_abar) {
    using MX = MxRing<P, N, kWide, LM>;
    const int L = r.L;
    const size_t gring = ((size_t)b * r.G + g) * L;
    const size_t hring = bh * L;
    const int t0 = count - W;
    const int bmod = base % L;
    auto slot = [&](int j) { return ring_slot(bmod, j, L); };
    const int last = count - 1;
    const int lr = lane & 15, lq = lane >> 4;
    MX m;
    m.j0 = j0;
    {
        const int sl = slot(lane < count ? lane : last);
        m.aj = r.a[hring + sl];
        m.dtj = r.dt[hring + sl];
    }
#pragma unroll
    for (int kb = 0; kb < MX::KB; ++kb) {
        const int c = MX::col(kb, lane);
        const int j = j0 + lr;
        m.ka[kb] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(r.k) +
                                                    (gring + slot(j < count ? j : last)) * N + c);
        m.qb[kb] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(r.q) +
                                                    (gring + slot(t0 + (lr < W ? lr : W - 1))) * N + c);
    }
    const auto vres = make_rsrc(static_cast<const uint16_t *>(r.v) + hring * P, (uint32_t)(L * P * 2));
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int j = j0 + 4 * lq + kk;
        const uint32_t row = (uint32_t)slot(j < count ? j : last) * P;
#pragma unroll
        for (int pw = 0; pw < MX::PW; ++pw)
            m.vw[kk][pw] = __builtin_amdgcn_raw_buffer_load_b32(vres, (row + 2 * MX::vword(pw, lane)) * 2, 0, 0);
    }
    if (lane >= count) {
        m.aj = 1.f;
        m.dtj = 0.f;
    }
    const f32x4 dk = m.dots(lane);
    f32x4 wv;
    float ab;
    m.weights_cols(lane, count, W, wv, ab);
    if (j0 == 0 && lane < kWide) s_abar[lane] = ab;
    m.term_cols(lane, dk, wv, s_r);
}

// A lane's share of one load step of the tile: CVEC elements of one row.
template <int ST, bool BF>
struct WideA;

template <>
struct WideA<ST_F32, false> {   // 4 floats
    f32x4 v;
    __device__ __forceinline__ void load(const void *S, size_t e) {
        v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(static_cast<const float *>(S) + e));
    }
    __device__ __forceinline__ void set(uint4 u) { v = __builtin_bit_cast(f32x4, u); }
    __device__ __forceinline__ f32x4 f32() const { return v; }
};
template <>
struct WideA<ST_BF16, false> {   // 4 bf16, widened
    u32x2 v;
    __device__ __forceinline__ void load(const void *S, size_t e) {
        v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(S) + e));
    }
    __device__ __forceinline__ f32x4 f32() const {
        return f32x4{bf16_bits_to_f32(v.x & 0xffffu), bf16_bits_to_f32(v.x >> 16), bf16_bits_to_f32(v.y & 0xffffu),
                     bf16_bits_to_f32(v.y >> 16)};
    }
};
template <>
struct WideA<ST_FP8, false> {   // 4 e4m3 codes, widened (unscaled)
    uint32_t v;
    __device__ __forceinline__ void load(const void *S, size_t e) {
        v = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(static_cast<const uint8_t *>(S) + e));
    }
    __device__ __forceinline__ f32x4 f32() const {
        float x[4];
        fp8x4_to_f32(v, x);
        return f32x4{x[0], x[1], x[2], x[3]};
    }
};
template <int ST>
struct WideA<ST, true> {   // 16 bytes: 8 bf16, or 16 e4m3 codes
    uint4 v;
    __device__ __forceinline__ void load(const void *S, size_t e) {
        const char *p = static_cast<const char *>(S) + e * (ST == ST_BF16 ? 2 : 1);
        const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
        v = uint4{w.x, w.y, w.z, w.w};
    }
    __device__ __forceinline__ void set(uint4 u) { v = u; }
    // e4m3: codes 8h..8h+7 as bf16 pairs (exact)
    __device__ __forceinline__ uint4 bf16_half(int h) const {
        const uint32_t w0 = h ? v.z : v.x, w1 = h ? v.w : v.y;
        return uint4{bf16_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false)),
                     bf16_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true)),
                     bf16_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false)),
                     bf16_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true))};
    }
};

template <int P, int N, int ST, int LM>
__global__ __launch_bounds__((WideShape<P, N, ST, LM>::NT)) void verify_wide_kernel(DecodeArgs args) {
    using WS = WideShape<P, N, ST, LM>;
    constexpr bool BF = WS::BF;
    constexpr int NTS = WS::NTS, CVEC = WS::CVEC, STEPS = WS::STEPS, TS = WS::TS, NR = WS::NR;
    using TE = typename std::conditional<BF, uint16_t, float>::type;   // LDS element of Q

    __shared__ __align__(16) TE s_Q[kWide][TS];    // the window's queries, Q[w][n]
    __shared__ float s_r[NR][kWide][P];
    __shared__ float s_abar[kWide];
    __shared__ __align__(16) uint32_t s_T[WS::COAL ? NTS / 64 : 1][16][WS::TROW];   // per-wavefront staging

    const RingView &r = args.r;
    const int W = args.W;
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int H = r.H, L = r.L;
    const int b = lid / H, h = lid % H;
    const int g = (h * r.G) / H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t bh = (size_t)b * H + h;
    const int p0 = 16 * wave;   // rows of a streaming wavefront

    // pointer pair first, then the tile rows (which do not depend on it)
    const int base = r.base[b];
    const int pos = r.pos[b];
    WideA<ST, BF> at[STEPS];
    uint4 raw[WS::COAL ? STEPS : 1];   // coalesced: load 2c + hf = rows 8hf + lane/8, bytes 128c + 16 (lane % 8)
    if (wave < NTS / 64) {
        if constexpr (WS::COAL) {
            const char *t = static_cast<const char *>(args.S) + (bh * (size_t)(P * N) + (size_t)p0 * N) * WS::ESZ;
#pragma unroll
            for (int i = 0; i < STEPS; ++i) {
                const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                    t + (size_t)(8 * (i & 1) + (lane >> 3)) * WS::RB + 128 * (i >> 1) + 16 * (lane & 7)));
                raw[i] = uint4{w.x, w.y, w.z, w.w};
            }
        } else {
            const size_t row = bh * (size_t)(P * N) + (size_t)(p0 + lr) * N;
#pragma unroll
            for (int st = 0; st < STEPS; ++st) at[st].load(args.S, row + (size_t)(4 * st + lg) * CVEC);
        }
    }
    const int count = pos - base;
    if (count < W) {  // uniform over the workgroup
        for (int i = tid; i < W * P; i += WS::NT) args.y[(((size_t)b * W + i / P) * H + h) * P + i % P] = __builtin_nanf("");
        if (tid == 0) raise_seq_error(r.err, b, REPLAY_SEQERR_TOO_FEW);
        return;
    }

    if (wave >= NTS / 64) {
        // The ring wavefront ends here, after the barrier that publishes its
        // terms; no path from its code reaches the tile registers' use, so
        // they stay free for it.
        const int blk = __builtin_amdgcn_readfirstlane(wave - NTS / 64);   // 16-entry block of the ring
        wide_ring_wave<P, N, LM>(r, lane, 16 * blk, b, g, bh, base, count, W, s_r[blk], s_abar);
        __syncthreads();
        return;
    }
    {
        // the queries: row w of Q is ring entry count-W+w (bf16), zero for w >= W;
        // 8 elements (16 bytes) a thread, every load issued before any is used
        const size_t gring = ((size_t)b * r.G + g) * L;
        const int bmod = base % L;
        constexpr int QP = kWide * N / 8, QI = (QP + NTS - 1) / NTS;
        uint4 qraw[QI];
#pragma unroll
        for (int i = 0; i < QI; ++i) {
            const int e = (i * NTS + tid < QP ? i * NTS + tid : QP - 1) * 8;
            const int w = e / N, n = e % N;
            qraw[i] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(r.q) +
                                                      (gring + ring_slot(bmod, count - W + (w < W ? w : W - 1), L)) * N + n);
        }
#pragma unroll
        for (int i = 0; i < QI; ++i) {
            if (i * NTS + tid < QP) {
                const int e = (i * NTS + tid) * 8;
                const int w = e / N, n = e % N;
                const uint4 u = w < W ? qraw[i] : uint4{0u, 0u, 0u, 0u};
                if constexpr (BF) {
                    *reinterpret_cast<uint4 *>(&s_Q[w][n]) = u;
                } else {
                    const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        s_Q[w][n + 2 * q] = bf16_bits_to_f32(wd[q] & 0xffffu);
                        s_Q[w][n + 2 * q + 1] = bf16_bits_to_f32(wd[q] >> 16);
                    }
                }
            }
        }
    }
    __syncthreads();

    {
        if constexpr (WS::COAL) {
            // chunk by chunk through this wavefront's buffer: lane (row lr,
            // group lg) of step st reads row lr, bytes 64 (st % 2) + 16 lg of
            // chunk st / 2 (a wavefront's own LDS accesses complete in order,
            // so the next chunk's writes follow this chunk's reads)
            uint32_t(*T)[WS::TROW] = s_T[wave];
#pragma unroll
            for (int c = 0; c < STEPS / 2; ++c) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
                    *reinterpret_cast<uint4 *>(&T[8 * hf + (lane >> 3)][4 * (lane & 7)]) = raw[2 * c + hf];
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                    at[2 * c + s2].set(*reinterpret_cast<const uint4 *>(&T[lr][16 * s2 + 4 * lg]));
            }
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const int c0 = (4 * st + lg) * CVEC;   // first column of this lane's load
            if constexpr (!BF) {
                const f32x4 a = at[st].f32();
                const f32x4 q = *reinterpret_cast<const f32x4 *>(&s_Q[lr][c0]);
#pragma unroll
                for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], q[t], acc, 0, 0, 0);
            } else if constexpr (ST == ST_BF16) {
                const uint4 q = *reinterpret_cast<const uint4 *>(&s_Q[lr][c0]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(at[st].v), as_bf16x8(q), acc, 0, 0, 0);
            } else {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const uint4 q = *reinterpret_cast<const uint4 *>(&s_Q[lr][c0 + 8 * hh]);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(at[st].bf16_half(hh)), as_bf16x8(q), acc,
                                                                  0, 0, 0);
                }
            }
        }
        // D[p0 + 4 lg + rr][w = lr]
        const int w = lr;
        if (w < W) {
            const float sc = (ST == ST_FP8) ? static_cast<const float *>(args.scale)[bh] : 1.0f;
            const float ab = s_abar[w];
            f32x4 o;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int p = p0 + 4 * lg + rr;
                float rt = s_r[0][w][p];
                if constexpr (NR == 2) rt += s_r[1][w][p];   // block 0 + block 1
                o[rr] = ab * (sc * acc[rr]) + rt;
            }
            *reinterpret_cast<f32x4 *>(&args.y[(((size_t)b * W + w) * H + h) * P + p0 + 4 * lg]) = o;
        }
    }
}

template <int P, int N, int ST>
static hipError_t launch_wide_st(const DecodeArgs &a, hipStream_t s) {
    const unsigned blocks = (unsigned)((size_t)a.r.B * a.r.H);
    if (a.r.L <= 16)
        verify_wide_kernel<P, N, ST, 16><<<blocks, WideShape<P, N, ST, 16>::NT, 0, s>>>(a);
    else
        verify_wide_kernel<P, N, ST, kMaxRing><<<blocks, WideShape<P, N, ST, kMaxRing>::NT, 0, s>>>(a);
    return hipGetLastError();
}

template <int P, int N>
static hipError_t launch_wide_pn(int st, const DecodeArgs &a, hipStream_t s) {
    switch (st) {
        case ST_F32: return launch_wide_st<P, N, ST_F32>(a, s);
        case ST_BF16: return launch_wide_st<P, N, ST_BF16>(a, s);
        case ST_FP8: return launch_wide_st<P, N, ST_FP8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

bool verify_wide_supported(int st, const DecodeArgs &a) {
    return a.r.io_bf16 && (st == ST_F32 || st == ST_BF16 || st == ST_FP8) && a.W >= 1 &&
           a.W <= kMaxWideWindow && a.W <= a.r.L;
}

hipError_t launch_verify_wide(int P, int N, int st, const DecodeArgs &a, hipStream_t s) {
    if (!verify_wide_supported(st, a)) return hipErrorInvalidValue;
    if (P == 16 && N == 16) return launch_wide_pn<16, 16>(st, a, s);
    if (P == 64 && N == 64) return launch_wide_pn<64, 64>(st, a, s);
    if (P == 64 && N == 128) return launch_wide_pn<64, 128>(st, a, s);
    if (P == 128 && N == 128) return launch_wide_pn<128, 128>(st, a, s);
    return hipErrorInvalidValue;
}

}  // namespace replay
