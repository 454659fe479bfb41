// ring_mx.h -- the ring part of the output-only route on the matrix cores
// (bf16 io): for the W newest entries t_w = count-W+w of one (sequence, head)
//     R[w][p] = sum_{j<=t_w} s_{j,t_w} (k_j . q_{t_w}) v_j[p],   abar_w = prod_{m<=t_w} a_m
// (page "ReplaySSM: Cachear Inputs, No Estado", section "Los dos caminos",
// eq. "Ruta solo salida", its sum over the buffer; s_{j,t} = dt_j
// prod_{j<m<=t} a_m, products taken left to right).
//
// Two small products, both in 16x16 MFMA tiles (lane l: row l%16, k-group
// l/16):
//   dots  D[j][w] = k_j . q_{t_w}     v_mfma_f32_16x16x32_bf16, A = k rows of
//                                     entries 16jb..16jb+15, B = the W queries
//                                     (columns w >= W are clamped copies, weighted 0)
//   term  R[w][p] = sum_j c[w][j] v_j[p],  c[w][j] = s_{j,t_w} D[j][w] (0 for j > t_w)
//                                     v_mfma_f32_16x16x4_f32, A = c, B = v rows
//                                     (a lane holds one bf16 pair: columns n of the
//                                     two products of a 32-wide block are p = 2n, 2n+1)
// The contraction slot k of the second product at lane (row, k) stands for
// entry 16jb + 4k + kk, which is where output register kk of the first
// product already holds D[j][w] for that lane, so c never moves between lanes.
// Segment weights are formed with lane = entry and handed over through LDS.
// bf16 products are exact in float32; only the order of the sums differs
// from a sequential evaluation.
#pragma once
#include "device_common.h"

namespace replay {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// One ring wavefront's share: the 16 entries j0..j0+15 (a 32-entry ring
// has two such wavefronts; their terms are added by the caller, block 0 +
// block 1).  IOB false: float32 ring operands; the dots then take
// v_mfma_f32_16x16x4_f32, eight per 32-column block (lane group g holds
// columns 32kb + 8g .. +7, product t takes column 32kb + 8g + t), and a
// lane's v values are float pairs.
template <int P, int N, int WM, int LM, bool IOB = true>
struct MxRing {
    static constexpr int KB = (N + 31) / 32;      // 32-column blocks of k . q
    static constexpr int PW = (P + 31) / 32;      // 32-column blocks of v, one bf16 pair per lane
    static constexpr int NR = LM / 16;            // ring wavefronts per (sequence, head)
    static_assert(LM % 16 == 0 && P % 16 == 0 && N % 16 == 0, "tile shape");

    // Operands, filled by the caller with raw bf16 bits (IOB) or floats.  Lane l = r + 16 g:
    int j0;                         // first entry of this wavefront's block
    uint4 ka[KB];                   // k_{j0 + r}[32kb + 8g .. +7]        (entries past the live ones: any finite row)
    uint4 qb[KB];                   // q_{t_min(r, W-1)}[32kb + 8g .. +7]
    uint32_t vw[4][PW];             // v_{j0 + 4g + kk}[32pw + 2r .. +1]   (same; pairs past P: any finite word)
    f32x4 kf[IOB ? 1 : KB][2];      // float32 io: the same k, q and v values as floats
    f32x4 qf[IOB ? 1 : KB][2];
    u32x2 vf[IOB ? 1 : 4][PW];
    float aj, dtj;                  // lane j (all LM entries): a_j, dt_j; 1 and 0 for j >= count

    // word index of lane l's v pair in block pw, clamped into the row
    static __device__ __forceinline__ int vword(int pw, int lane) {
        const int w = 16 * pw + (lane & 15);
        return w < P / 2 ? w : P / 2 - 1;
    }

    static __device__ __forceinline__ float vval(uint32_t word, int half) {
        return half ? __uint_as_float(word & 0xffff0000u) : __uint_as_float(word << 16);
    }

    static __device__ __forceinline__ int col(int kb, int lane) {
        const int c = 32 * kb + 8 * (lane >> 4);
        return c < N ? c : 0;
    }

    __device__ __forceinline__ f32x4 dots(int lane) const {
        f32x4 dk = {0.f, 0.f, 0.f, 0.f};
        if constexpr (!IOB) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    // columns past N (only when N < 32) count zero
                    const float a = 32 * kb + 8 * (lane >> 4) < N ? kf[kb][t >> 2][t & 3] : 0.f;
                    dk = __builtin_amdgcn_mfma_f32_16x16x4f32(a, qf[kb][t >> 2][t & 3], dk, 0, 0, 0);
                }
            return dk;
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            uint4 a = ka[kb];
            if (32 * kb + 8 * (lane >> 4) >= N) a = uint4{0u, 0u, 0u, 0u};   // only when N < 32
            dk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(qb[kb]), dk, 0, 0, 0);
        }
        return dk;
    }

    // s_sw[w][j] = s_{j,t_w} (0 for j > t_w or j >= count) for this block's
    // entries; s_abar[w] = abar_{t_w} from the block-0 wavefront.  A window
    // of W < WM positions leaves columns w >= W at zero (t_w = count-W+w).
    __device__ __forceinline__ void weights(int lane, int count, float *s_abar, float (*s_sw)[LM],
                                            int W = WM) const {
        const int t0 = count - W;
        float sw[WM], ab[WM];
        float prod = dtj, run = 1.f;
        // entries before the window (a loop over the wave-uniform count),
        // then the window's W entries, each taking its weights once formed
        for (int m = 0; m < t0; ++m) {
            const float am = bcast(aj, m);
            if (m > lane) prod *= am;
            run *= am;
        }
#pragma unroll
        for (int w = 0; w < WM; ++w) {
            sw[w] = ab[w] = 0.f;
            if (w < W && t0 + w >= 0) {   // (count >= W at every call: the second test never fails)
                const int m = t0 + w;
                const float am = bcast(aj, m);
                if (m > lane) prod *= am;
                run *= am;
                sw[w] = prod;
                ab[w] = run;
            }
        }
        if (lane >= j0 && lane < j0 + 16) {
#pragma unroll
            for (int w = 0; w < WM; ++w) s_sw[w][lane] = lane <= t0 + w ? sw[w] : 0.f;
        }
        if (j0 == 0 && lane == 0) {
#pragma unroll
            for (int w = 0; w < WM; ++w) s_abar[w] = ab[w];
        }
    }

    // The same weights in the term's operand layout, without LDS: lane
    // (w = lane%16, group lq) forms s_{j,t_w} for its four entries j =
    // j0+4lq+kk and abar_{t_w}, multiplying the same factors in the same
    // order as weights() (dt_j, then a_m for j < m <= t_w), so the values are
    // identical.  Columns w >= W get zero weights and abar.
    __device__ __forceinline__ void weights_cols(int lane, int count, int W, f32x4 &wv, float &abar) const {
        const int w = lane & 15, jb = j0 + 4 * (lane >> 4);
        const int t = count - W + w;
        float pr[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) pr[kk] = __shfl(dtj, jb + kk);
        float run = 1.f;
#pragma unroll
        for (int m = 0; m < LM; ++m) {
            if (m < count) {
                const float am = bcast(aj, m);
                const bool in_t = m <= t;
                run = in_t ? run * am : run;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    if (in_t && m > jb + kk) pr[kk] *= am;
            }
        }
        const bool valid = w < W;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) wv[kk] = valid && jb + kk <= t ? pr[kk] : 0.f;
        abar = valid ? run : 0.f;
    }

    // The ring term with weights already in the operand layout (weights_cols).
    __device__ __forceinline__ void term_cols(int lane, f32x4 dk, f32x4 wv, float (*s_r)[P]) const {
        const int lr = lane & 15, lq = lane >> 4;
        const f32x4 cf = wv * dk;
        term_coeffs(lr, lq, cf, s_r);
    }

    // s_r[w][p] = this block's part of R[w][p]; reads the weights this
    // wavefront wrote to s_sw (other lanes' writes: wave_lds_sync first)
    __device__ __forceinline__ void term(int lane, f32x4 dk, float (*s_r)[P], const float (*s_sw)[LM]) const {
        const int lr = lane & 15, lq = lane >> 4;
        wave_lds_sync();
        const f32x4 wv = *reinterpret_cast<const f32x4 *>(&s_sw[lr < WM ? lr : 0][j0 + 4 * lq]);
        const f32x4 cf = lr < WM ? wv * dk : f32x4{0.f, 0.f, 0.f, 0.f};
        term_coeffs(lr, lq, cf, s_r);
    }

    // s_r[w][p] = sum_j cf[w][j] v_j[p] from the coefficients in the first
    // product's output layout
    __device__ __forceinline__ void term_coeffs(int lr, int lq, f32x4 cf, float (*s_r)[P]) const {
        // column n of block (pw, half) is p = 32pw + 2n + half
#pragma unroll
        for (int pw = 0; pw < PW; ++pw)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const float vv = IOB ? vval(vw[kk][pw], half) : __uint_as_float(vf[IOB ? 0 : kk][pw][half]);
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(cf[kk], vv, acc, 0, 0, 0);
                }
                const int p = 32 * pw + 2 * lr + half;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int w = 4 * lq + rr;
                    if (w < WM && p < P) s_r[w][p] = acc[rr];
                }
            }
    }
};

}  // namespace replay
