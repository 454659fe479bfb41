// gdn.hip -- Gated DeltaNet layers on the replay path, for gfx950.
//
// The pages name Gated DeltaNet as the second layer type the replay serves
// (page "ReplaySSM: Cache SSM Inputs, Not State", Abstract; page "ReplaySSM:
// que cambia en los modelos hibridos de IA", section "Una integracion
// concreta no cubre todas las opciones") without its equation.  The rule is
// the published gated delta rule, with S a P x N (value x key) matrix per
// (sequence, head) and the ring's dt slot holding beta_t, its a slot alpha_t:
//
//   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   y_t = S_t q_t
//
// Unrolled from the checkpoint S0 over ring entries 1..t (A_m = alpha_m (I -
// beta_m k_m k_m^T)):  S_t q_t = S0 w_0 + sum_j beta_j v_j (k_j . w_j), where
// w_t = q_t and w_{m-1} = A_m w_m.  So the output-only route of this layer
// runs a backward chain over the ring (2N multiply-adds an entry) and then
// one pass over S0 with w_0, the pages' "one read of the checkpoint, no state
// write" (page "ReplaySSM: Cachear Inputs, No Estado", section "Los dos
// caminos", eq. "Ruta solo salida", in this layer's form).  The fold applies
// the rule entry after entry to every row of S0 and writes it once.
//
// Kernels
//   gdn_verify_kernel  W newest entries (W = 1: decode) scored against one read
//                      of S0.  A chain wavefront stages the entries' k and v in
//                      LDS, runs the W backward chains (64-lane dot products)
//                      and the ring term, and hands w_0 over through LDS; the
//                      streaming wavefronts hold the tile (16-byte float32
//                      chunks, loaded before the chain ends) and take its dot
//                      products with the W vectors w_0.
//   gdn_fold_kernel    eight lanes a row (interleaved 16-byte pieces: every load
//                      and store instruction covers whole 128-byte lines), the
//                      tile in registers; an entry costs a row dot, three lane
//                      exchanges and two operations an element.  With EMIT it
//                      is the eager step of this layer (one entry from the
//                      call, y = S_t q_t).
#include "decode_impl.h"
#include "wide_mx.h"

namespace replay {

// ---------------------------------------------------------------------------
// Output-only route: decode (W = 1) and verify (W <= kMaxWindow)

// The decode kernel's shape: PR of the head's P rows per workgroup (a 128 x
// 128 float32 head is streamed by two workgroups of 64 rows, 4 + 1 wavefronts
// each; six fit a compute unit where three of 8 + 1 did), or HPW whole heads
// of one group (low-precision copies: their small tiles streamed as one
// taller tile, one chain wavefront a head).
template <int P, int N, int LM, bool IOB, int PR, int ST, int HPW>
struct GdnShape {
    static_assert(P % PR == 0 && (HPW == 1 || PR == P), "row blocks of one head, or whole heads");
    using Sh = DecodeShape<PR * HPW, N, ST, 1>;
    static constexpr int SPL = P / PR;            // workgroups a head
    static constexpr int NTS = Sh::NTS;           // streaming threads
    static constexpr int NT = NTS + 64 * HPW;     // + a chain wavefront a head
};

// Rows 0..count-1 (count <= ROWS) of COLS io elements each, row j read from
// elements col0 .. col0 + COLS of ring row `first + ring_slot(bmod, j, L)` of
// `src` (rows of RS elements), widened into s[j][0..COLS): 16-byte pieces (8
// bf16 or 4 floats) over NTHR threads, in batches of up to 8 pieces a thread
// whose loads are all issued before any is stored (one memory latency a
// batch, a bounded number of registers).
template <int ROWS, int COLS, int NTHR, bool IOB, int RS = COLS>
__device__ __forceinline__ void gdn_stage_rows(const void *src, size_t first, int bmod, int L, int count, int tid,
                                               float (*s)[COLS], int col0 = 0) {
    auto slot = [bmod, L](int j) { return ring_slot(bmod, j, L); };
    constexpr int PE = IOB ? 8 : 4;                        // elements a piece
    constexpr int PIECES = ROWS * COLS / PE;
    constexpr int PER = (PIECES + NTHR - 1) / NTHR;        // pieces a thread
    constexpr int BATCH = PER < 8 ? PER : 8;
    static_assert(COLS % PE == 0 && PER % BATCH == 0, "rows of whole pieces");
#pragma unroll
    for (int i0 = 0; i0 < PER; i0 += BATCH) {
        uint4 raw[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            const int c = tid + (i0 + i) * NTHR;
            const int j = c / (COLS / PE), n = (c % (COLS / PE)) * PE;
            if (c < PIECES && j < count) {
                const size_t e = (first + slot(j)) * RS + col0 + n;
                if constexpr (IOB)
                    raw[i] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(src) + e);
                else
                    raw[i] = *reinterpret_cast<const uint4 *>(static_cast<const float *>(src) + e);
            }
        }
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            const int c = tid + (i0 + i) * NTHR;
            const int j = c / (COLS / PE), n = (c % (COLS / PE)) * PE;
            if (c < PIECES && j < count) {
                if constexpr (IOB) {
                    const uint32_t u[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        s[j][n + 2 * e] = bf16_bits_to_f32(u[e] & 0xffffu);
                        s[j][n + 2 * e + 1] = bf16_bits_to_f32(u[e] >> 16);
                    }
                } else {
                    *reinterpret_cast<f32x4 *>(&s[j][n]) =
                        f32x4{__uint_as_float(raw[i].x), __uint_as_float(raw[i].y), __uint_as_float(raw[i].z),
                              __uint_as_float(raw[i].w)};
                }
            }
        }
    }
}

// Sum over the 64 lanes of a wavefront, returned in every lane: DPP steps
// within each row of 16 lanes, then the four row sums read out by readlane
// (no LDS round trip, as a cross-row shuffle would take).
__device__ __forceinline__ float gdn_wave_sum(float x) {
#pragma unroll
    for (int bit = 3; bit >= 0; --bit) x += lane_partner(x, bit);   // row sums, in every lane of the row
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return (r0 + r1) + (r2 + r3);
}

// The chain wavefront: entries 0..count-1 of (b, h); window position w is
// entry t_w = count - W + w.  For the WM positions w_lo .. w_lo + WM - 1
// below W, writes s_w0[w][n] = w_0 of position w and, for the PR rows
// p0 .. p0 + PR, s_r[w][p - p0] = sum_{j<=t_w} beta_j (k_j . w_j) v_j[p].
// STAGE: this wavefront stages the entries' k and v rows itself (else the
// caller has staged them and synchronised); ZROW: rows w_lo.. of s_w0 past
// W are written as zeros.  QS: the row stride of s_w0.
template <int P, int N, int WM, int LM, bool IOB, int PR, bool STAGE = true, bool ZROW = false, int QS = N>
__device__ __forceinline__ void gdn_chain_wave(const RingView &r, int lane, int b, int g, size_t bh, int base,
                                               int count, int W, int p0, float (*s_k)[N], float (*s_v)[PR],
                                               float (*s_w0)[QS], float (*s_r)[PR], int w_lo = 0) {
    constexpr int E = (N + 63) / 64, VR = (PR + 63) / 64;
    const int L = r.L;
    const int bmod = base % L;
    auto slot = [&](int j) { return ring_slot(bmod, j, L); };
    const size_t gring = ((size_t)b * r.G + g) * L;
    const size_t hring = bh * L;

    // every load first: lane m's alpha_m and beta_m, the window's queries, the
    // entries' k and v rows (staged in LDS)
    float aj = 1.f, bj = 0.f;
    if (lane < count) {
        aj = r.a[dta_index(b, bh, r.H, L, slot(lane))];
        bj = r.dt[dta_index(b, bh, r.H, L, slot(lane))];
    }
    float wv[WM][E];
#pragma unroll
    for (int w = 0; w < WM; ++w) {
        const int t = count - W + (w_lo + w < W ? w_lo + w : W - 1);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int n = lane + 64 * e;
            float x = 0.f;
            if (n < N) {
                if constexpr (IOB)
                    x = bf16_bits_to_f32(static_cast<const uint16_t *>(r.q)[(gring + slot(t)) * N + n]);
                else
                    x = static_cast<const float *>(r.q)[(gring + slot(t)) * N + n];
            }
            wv[w][e] = x;
        }
    }
    if constexpr (STAGE) {
        gdn_stage_rows<LM, N, 64, IOB>(r.k, gring, bmod, L, count, lane, s_k);
        gdn_stage_rows<LM, PR, 64, IOB, P>(r.v, hring, bmod, L, count, lane, s_v, p0);
        wave_lds_sync();   // every lane's k and v rows are in LDS
    }

    float acc[WM][VR];
#pragma unroll
    for (int w = 0; w < WM; ++w)
#pragma unroll
        for (int rr = 0; rr < VR; ++rr) acc[w][rr] = 0.f;
    // entries from the newest down: position w takes entry m once m <= t_w
#pragma unroll
    for (int m = LM - 1; m >= 0; --m) {
        if (m < count) {   // uniform
            const float am = bcast(aj, m), bm = bcast(bj, m);
            float km[E], vm[VR];
#pragma unroll
            for (int e = 0; e < E; ++e) km[e] = lane + 64 * e < N ? s_k[m][lane + 64 * e] : 0.f;
#pragma unroll
            for (int rr = 0; rr < VR; ++rr) vm[rr] = lane + 64 * rr < PR ? s_v[m][lane + 64 * rr] : 0.f;
#pragma unroll
            for (int w = 0; w < WM; ++w) {
                if (w_lo + w < W && m <= count - W + w_lo + w) {   // uniform
                    float d = 0.f;
#pragma unroll
                    for (int e = 0; e < E; ++e) d = fmaf(km[e], wv[w][e], d);
                    d = gdn_wave_sum(d);             // k_m . w_m, in every lane
                    const float c = bm * d;
#pragma unroll
                    for (int rr = 0; rr < VR; ++rr) acc[w][rr] = fmaf(c, vm[rr], acc[w][rr]);
#pragma unroll
                    for (int e = 0; e < E; ++e) wv[w][e] = am * fmaf(-c, km[e], wv[w][e]);   // w_{m-1} = A_m w_m
                }
            }
        }
    }
#pragma unroll
    for (int w = 0; w < WM; ++w) {
        if (w_lo + w < W) {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (lane + 64 * e < N) s_w0[w_lo + w][lane + 64 * e] = wv[w][e];
#pragma unroll
            for (int rr = 0; rr < VR; ++rr)
                if (lane + 64 * rr < PR) s_r[w_lo + w][lane + 64 * rr] = acc[w][rr];
        } else if constexpr (ZROW) {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (lane + 64 * e < N) s_w0[w_lo + w][lane + 64 * e] = 0.f;
        }
    }
}

// ST: the state the outputs read -- the float32 checkpoint, or a bf16 / e4m3
// / MX FP4 copy of it (page "ReplaySSM: Cache SSM Inputs, Not State",
// Abstract: a low-precision checkpoint serves the outputs).  A copy's values
// are widened exactly and dotted with the float32 w_0; e4m3 sums take the
// head's scale, FP4 sums each chunk's block scale (exact powers of two).
template <int P, int N, int LM, bool IOB, int PR, int ST, int HPW>
__global__ __launch_bounds__((GdnShape<P, N, LM, IOB, PR, ST, HPW>::NT)) void gdn_verify_kernel(DecodeArgs args) {
    using GS = GdnShape<P, N, LM, IOB, PR, ST, HPW>;
    using Sh = typename GS::Sh;
    constexpr int VEC = Sh::VEC, NTS = Sh::NTS, ITER = Sh::ITER, LPR = Sh::LPR, RPI = Sh::RPI;
    using RR = RowReduce<ITER, LPR>;
    static_assert(ST != ST_F32 || VEC == 4, "float32 chunks");

    __shared__ __align__(16) float s_k[HPW][LM][N];
    __shared__ __align__(16) float s_v[HPW][LM][PR];
    __shared__ __align__(16) float s_w0[HPW][1][N];
    __shared__ float s_r[HPW][1][PR];

    const RingView &r = args.r;
    // consecutive workgroups: the row blocks of a head (or the head pairs),
    // then the heads of a group (same compute die, whose L2 holds the
    // group's k rows)
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int H = r.H;
    const int hb = lid / GS::SPL, p0 = (lid % GS::SPL) * PR;   // (HPW > 1: SPL = 1, p0 = 0)
    const int b = hb / (H / HPW), h0 = (hb % (H / HPW)) * HPW;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t bh0 = (size_t)b * H + h0;
    const size_t tile = bh0 * (size_t)(P * N) + (size_t)p0 * N;

    const int base = r.base[b];
    const int pos = r.pos[b];
    const int count = pos - base;
    Chunk<ST, VEC> ch[ITER];
    if (wave < NTS / 64) {
#pragma unroll
        for (int i = 0; i < ITER; ++i) {
            if constexpr (ST == ST_FP4)
                ch[i].load_mx(args.S, args.scale, tile + (size_t)(i * NTS + tid) * VEC);
            else
                ch[i].load(args.S, tile + (size_t)(i * NTS + tid) * VEC);
        }
    }
    if (count < 1) {   // uniform over the workgroup
        for (int i = tid; i < HPW * PR; i += GS::NT) args.y[(bh0 + i / PR) * P + p0 + i % PR] = __builtin_nanf("");
        if (tid == 0) raise_seq_error(r.err, b, REPLAY_SEQERR_TOO_FEW);
        return;
    }
    if (wave >= NTS / 64) {
        const int hl = wave - NTS / 64;
        const int h = h0 + hl;
        gdn_chain_wave<P, N, 1, LM, IOB, PR>(r, lane, b, (h * r.G) / H, bh0 + hl, base, count, 1, p0, s_k[hl],
                                             s_v[hl], s_w0[hl], s_r[hl]);
    }
    __syncthreads();
    if (wave >= NTS / 64) return;

    // S0 w_0: partial sums over this lane's chunks (each chunk's rows are of
    // one head: w_0 of that head), then the row reduction across the LPR lanes
    const int col0 = (tid % LPR) * VEC;
    float part[ITER][1];
#pragma unroll
    for (int i = 0; i < ITER; ++i) {
        const int hl = HPW == 1 ? 0 : (i * RPI + tid / LPR) / PR;
        if constexpr (ST == ST_F32) {
            const f32x4 q = *reinterpret_cast<const f32x4 *>(&s_w0[hl][0][col0]);
            const f32x4 x = ch[i].raw;
            part[i][0] = fmaf(x.x, q.x, fmaf(x.y, q.y, fmaf(x.z, q.z, x.w * q.w)));
        } else {
            float x[VEC];
            ch[i].widen(x, 1.0f);   // the codes' values, unscaled
            float acc = 0.f;
#pragma unroll
            for (int e4 = 0; e4 < VEC / 4; ++e4) {
                const f32x4 q = *reinterpret_cast<const f32x4 *>(&s_w0[hl][0][col0 + 4 * e4]);
                acc = fmaf(x[4 * e4], q.x, acc);
                acc = fmaf(x[4 * e4 + 1], q.y, acc);
                acc = fmaf(x[4 * e4 + 2], q.z, acc);
                acc = fmaf(x[4 * e4 + 3], q.w, acc);
            }
            if constexpr (ST == ST_FP4) acc = ldexpf(acc, ch[i].se);   // the block's scale, exact
            part[i][0] = acc;
        }
    }
    RR::template run<1>(part, lane);
    if (RR::writer(lane)) {
        const int hi = RR::halving_index(lane);
#pragma unroll
        for (int e = 0; e < RR::FINAL; ++e) {
            const int row = (e + RR::FINAL * hi) * RPI + tid / LPR;   // of the HPW stacked row blocks
            const int hl = HPW == 1 ? 0 : row / PR, p = HPW == 1 ? row : row % PR;
            const float sc = ST == ST_FP8 ? static_cast<const float *>(args.scale)[bh0 + hl] : 1.0f;   // e4m3 head scale
            args.y[(bh0 + hl) * P + p0 + p] = sc * part[e][0] + s_r[hl][0][p];
        }
    }
}

template <int P, int N, int ST, int LM, int PR, int HPW>
static hipError_t launch_gdn_decode_lm(const DecodeArgs &a, hipStream_t s) {
    const unsigned blocks = (unsigned)((size_t)a.r.B * a.r.H * (P / PR) / HPW);
    if (a.r.io_bf16)
        gdn_verify_kernel<P, N, LM, true, PR, ST, HPW><<<blocks, GdnShape<P, N, LM, true, PR, ST, HPW>::NT, 0, s>>>(a);
    else
        gdn_verify_kernel<P, N, LM, false, PR, ST, HPW><<<blocks, GdnShape<P, N, LM, false, PR, ST, HPW>::NT, 0, s>>>(a);
    return hipGetLastError();
}

// Float32 and bf16 tiles of 128 rows: two workgroups of 64 (with whole heads
// the copy kernels took 78 to 99 registers, three or four workgroups to a
// compute unit; bf16 85.9 -> 64.7 us a launch at B=256 H=32).  e4m3 and FP4
// copies: two heads of a group a workgroup, whole (their 8 and 16 KiB tiles
// stream in less time than a head's chain takes).
template <int P, int N, int ST, int LM>
static hipError_t launch_gdn_decode_st(const DecodeArgs &a, hipStream_t s) {
    constexpr bool PAIR = ST == ST_FP8 || ST == ST_FP4;
    if (PAIR && (a.r.H / a.r.G) % 2 == 0) return launch_gdn_decode_lm<P, N, ST, LM, P, 2>(a, s);
    constexpr int PR = P == 128 && !PAIR ? 64 : P;
    return launch_gdn_decode_lm<P, N, ST, LM, PR, 1>(a, s);
}

template <int P, int N, int ST>
static hipError_t launch_gdn_decode_l(const DecodeArgs &a, hipStream_t s) {
    if (a.r.L <= 16) return launch_gdn_decode_st<P, N, ST, 16>(a, s);
    return launch_gdn_decode_st<P, N, ST, kMaxRing>(a, s);
}

template <int P, int N>
static hipError_t launch_gdn_decode_pn(int st, const DecodeArgs &a, hipStream_t s) {
    switch (st) {
        case ST_F32: return launch_gdn_decode_l<P, N, ST_F32>(a, s);
        case ST_BF16: return launch_gdn_decode_l<P, N, ST_BF16>(a, s);
        case ST_FP8: return launch_gdn_decode_l<P, N, ST_FP8>(a, s);
        case ST_FP4: return launch_gdn_decode_l<P, N, ST_FP4>(a, s);
        default: return hipErrorInvalidValue;
    }
}

// The chains of eight window positions w_lo .. w_lo + 7 in one wavefront,
// positions on the wavefront's 16-lane rows: lane (row rw, column c) holds
// elements NE c .. NE c + NE - 1 of positions rw and rw + 4 (w vectors and the
// ring term's rows VR c .. VR c + VR - 1), so an entry's dot k_m . w_m is a sum
// over the 16 lanes of a row (DPP steps, no cross-row traffic).  A position
// not yet reached by entry m (m > t_w), or past W, takes alpha = 1, beta = 0
// for it: w and the ring term stay unchanged exactly.  Every lane stages the
// entries' k and v rows (stride 64 threads) as gdn_chain_wave does; rows of
// s_w0 past W are written as zeros.  The ring term covers rows r0 .. r0 + PR
// of the head.  The w_0 rows are written after a workgroup barrier (s_w0 may
// overlay s_k, which every chain wavefront reads until then); the caller's
// other wavefronts take that barrier too.
template <int P, int N, int LM, bool IOB, int QS, int PR>
__device__ __forceinline__ void gdn_chain_rows(const RingView &r, int lane, int b, int g, size_t bh, int base,
                                               int count, int W, int w_lo, int r0, float (*s_k)[N],
                                               float (*s_v)[PR], float (*s_w0)[QS], float (*s_r)[PR]) {
    constexpr int NE = N / 16, VR = PR / 16, PPR = 2;   // elements, outputs, positions of a lane
    static_assert(N % 16 == 0 && PR % 16 == 0, "whole 16-lane rows");
    const int L = r.L;
    const int bmod = base % L;
    auto slot = [&](int j) { return ring_slot(bmod, j, L); };
    const size_t gring = ((size_t)b * r.G + g) * L;
    const int rw = lane >> 4, c = lane & 15;

    float aj = 1.f, bj = 0.f;
    if (lane < count) {
        aj = r.a[dta_index(b, bh, r.H, L, slot(lane))];
        bj = r.dt[dta_index(b, bh, r.H, L, slot(lane))];
    }
    int gw[PPR];
    float wv[PPR][NE];
#pragma unroll
    for (int s = 0; s < PPR; ++s) {
        gw[s] = w_lo + rw + 4 * s;
        const int t = count - W + (gw[s] < W ? gw[s] : W - 1);
        const size_t q0 = (gring + slot(t)) * N + NE * c;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            if constexpr (IOB)
                wv[s][e] = bf16_bits_to_f32(static_cast<const uint16_t *>(r.q)[q0 + e]);
            else
                wv[s][e] = static_cast<const float *>(r.q)[q0 + e];
        }
    }
    gdn_stage_rows<LM, N, 64, IOB>(r.k, gring, bmod, L, count, lane, s_k);
    gdn_stage_rows<LM, PR, 64, IOB, P>(r.v, bh * L, bmod, L, count, lane, s_v, r0);
    wave_lds_sync();   // every lane's k and v rows are in LDS

    float acc[PPR][VR];
#pragma unroll
    for (int s = 0; s < PPR; ++s)
#pragma unroll
        for (int i = 0; i < VR; ++i) acc[s][i] = 0.f;
    // the entries from the newest down (unrolled over the ring's bound, uniform guards)
#pragma unroll
    for (int m = LM - 1; m >= 0; --m) {
      if (m < count) {
        const float am = bcast(aj, m), bm = bcast(bj, m);
        float km[NE], vm[VR];
#pragma unroll
        for (int e = 0; e < NE; ++e) km[e] = s_k[m][NE * c + e];
#pragma unroll
        for (int i = 0; i < VR; ++i) vm[i] = s_v[m][VR * c + i];
#pragma unroll
        for (int s = 0; s < PPR; ++s) {
            if (w_lo + 4 * s >= W) continue;   // uniform: no position of this slot is in the window
            const bool act = gw[s] < W && m <= count - W + gw[s];
            const float as = act ? am : 1.f, bs = act ? bm : 0.f;
            float d0 = 0.f, d1 = 0.f;   // two partial sums: a shorter dependent chain
#pragma unroll
            for (int e = 0; e < NE; e += 2) {
                d0 = fmaf(km[e], wv[s][e], d0);
                if (e + 1 < NE) d1 = fmaf(km[e + 1], wv[s][e + 1], d1);
            }
            float d = d0 + d1;
#pragma unroll
            for (int bit = 3; bit >= 0; --bit) d += lane_partner(d, bit);   // over the row's 16 lanes
            const float cf = bs * d;
#pragma unroll
            for (int i = 0; i < VR; ++i) acc[s][i] = fmaf(cf, vm[i], acc[s][i]);
#pragma unroll
            for (int e = 0; e < NE; ++e) wv[s][e] = as * fmaf(-cf, km[e], wv[s][e]);   // w_{m-1} = A_m w_m
        }
      }
    }
#pragma unroll
    for (int s = 0; s < PPR; ++s) {
        if (gw[s] < W) {
#pragma unroll
            for (int i = 0; i < VR; ++i) s_r[gw[s]][VR * c + i] = acc[s][i];
        }
    }
    __syncthreads();   // every chain wavefront of the workgroup is done with s_k, which s_w0 overlays
#pragma unroll
    for (int s = 0; s < PPR; ++s) {
        const bool live = gw[s] < W;
#pragma unroll
        for (int e = 0; e < NE; ++e) s_w0[gw[s]][NE * c + e] = live ? wv[s][e] : 0.f;
    }
}

// ---------------------------------------------------------------------------
// Windows past the register kernel's 8 (up to 16): S0 W_0^T on the matrix
// cores.  The streaming wavefronts are the matrix-core verify's (wide_mx.h:
// one per 16 rows, coalesced tile reads transposed per wavefront in LDS,
// v_mfma_f32_16x16x4_f32 against float32 query rows), the query rows being
// the window positions' w_0 from the chains; two chain wavefronts run eight
// positions each.  Each stages every k and v row into the one buffer itself
// (the two write the same values), so neither waits for the other.

// PR of the head's P rows per workgroup (128-row heads: two workgroups of
// 64, each running both chain wavefronts for its own rows).  The w_0 rows
// overlay the staged k rows once every chain has finished reading them.
template <int P, int N, int ST, int LM, int PR>
struct GdnWideShape : WideTile<PR, N, ST> {
    static constexpr int SPL = P / PR;                     // workgroups a head
    static constexpr int NC = kWide / 8;                   // chain wavefronts, 8 positions each
    static constexpr int NT = WideTile<PR, N, ST>::NTS + 64 * NC;
    static constexpr int TSF = N + 4;                      // LDS row stride of the w_0 rows, in floats
    static constexpr int KQ = LM * N > kWide * TSF ? LM * N : kWide * TSF;   // floats of the k / w_0 buffer
};

template <int P, int N, int ST, int LM, bool IOB, int PR>
__global__ __launch_bounds__((GdnWideShape<P, N, ST, LM, PR>::NT)) void gdn_wide_kernel(DecodeArgs args) {
    using WS = GdnWideShape<P, N, ST, LM, PR>;
    constexpr int NTS = WS::NTS, TSF = WS::TSF;

    __shared__ __align__(16) float s_kq[WS::KQ];        // the entries' k rows, then w_0 of each window position
    __shared__ float s_r[kWide][PR];
    __shared__ __align__(16) float s_v[LM][PR];
    __shared__ __align__(16) uint32_t s_T[WS::COAL ? NTS / 64 : 1][16][WS::TROW];   // per-wavefront staging
    float (*s_k)[N] = reinterpret_cast<float (*)[N]>(s_kq);
    float (*s_Qf)[TSF] = reinterpret_cast<float (*)[TSF]>(s_kq);

    const RingView &r = args.r;
    const int W = args.W;
    // consecutive workgroups: the row blocks of a head, then the heads of a group
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int H = r.H;
    const int hb = lid / WS::SPL, r0 = (lid % WS::SPL) * PR;
    const int b = hb / H, h = hb % H;
    const int g = (h * r.G) / H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t bh = (size_t)b * H + h;
    const int p0 = r0 + 16 * wave;   // rows of a streaming wavefront

    const int base = r.base[b];
    const int pos = r.pos[b];
    WideRows<P, N, ST> rows;
    if (wave < NTS / 64) rows.load(args.S, bh * (size_t)(P * N), p0, lane, args.scale);
    const int count = pos - base;
    if (count < W) {  // uniform over the workgroup
        for (int i = tid; i < W * PR; i += WS::NT)
            args.y[(((size_t)b * W + i / PR) * H + h) * P + r0 + i % PR] = __builtin_nanf("");
        if (tid == 0) raise_seq_error(r.err, b, REPLAY_SEQERR_TOO_FEW);
        return;
    }
    if (wave >= NTS / 64) {
        // chain wavefront c: positions 8c .. 8c + 7 (two barriers inside and here)
        const int c = __builtin_amdgcn_readfirstlane(wave - NTS / 64);
        gdn_chain_rows<P, N, LM, IOB, TSF, PR>(r, lane, b, g, bh, base, count, W, 8 * c, r0, s_k, s_v, s_Qf, s_r);
        __syncthreads();   // the w_0 rows and the ring terms
        return;
    }
    rows.transpose(s_T[WS::COAL ? wave : 0], lane);
    __syncthreads();   // the chains are done with the k rows
    __syncthreads();   // the w_0 rows and the ring terms
    const uint8_t *rsc = static_cast<const uint8_t *>(args.scale) + (bh * P + p0 + 4 * lg) * WS::NB;   // FP4 rows
    const f32x4 acc = rows.dot_f32q(s_Qf, lane, rsc);
    // D[p0 + 4 lg + rr][w = lr]
    const int w = lr;
    if (w < W) {
        const float sc = (ST == ST_FP8) ? static_cast<const float *>(args.scale)[bh] : 1.0f;
        f32x4 o;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) o[rr] = sc * acc[rr] + s_r[w][p0 - r0 + 4 * lg + rr];
        *reinterpret_cast<f32x4 *>(&args.y[(((size_t)b * W + w) * H + h) * P + p0 + 4 * lg]) = o;
    }
}

template <int P, int N, int ST, int LM, int PR>
static hipError_t launch_gdn_wide_lm(const DecodeArgs &a, hipStream_t s) {
    const unsigned blocks = (unsigned)((size_t)a.r.B * a.r.H * (P / PR));
    if (a.r.io_bf16)
        gdn_wide_kernel<P, N, ST, LM, true, PR><<<blocks, GdnWideShape<P, N, ST, LM, PR>::NT, 0, s>>>(a);
    else
        gdn_wide_kernel<P, N, ST, LM, false, PR><<<blocks, GdnWideShape<P, N, ST, LM, PR>::NT, 0, s>>>(a);
    return hipGetLastError();
}

template <int P, int N, int ST>
static hipError_t launch_gdn_wide_st(const DecodeArgs &a, hipStream_t s) {
    constexpr int PR = P == 128 ? 64 : P;
    if (a.r.L <= 16) return launch_gdn_wide_lm<P, N, ST, 16, PR>(a, s);
    return launch_gdn_wide_lm<P, N, ST, kMaxRing, PR>(a, s);
}

template <int P, int N>
static hipError_t launch_gdn_wide_pn(int st, const DecodeArgs &a, hipStream_t s) {
    switch (st) {
        case ST_F32: return launch_gdn_wide_st<P, N, ST_F32>(a, s);
        case ST_BF16: return launch_gdn_wide_st<P, N, ST_BF16>(a, s);
        case ST_FP8: return launch_gdn_wide_st<P, N, ST_FP8>(a, s);
        case ST_FP4: return launch_gdn_wide_st<P, N, ST_FP4>(a, s);
        default: return hipErrorInvalidValue;
    }
}

static hipError_t launch_gdn_wide(int P, int N, int st, const DecodeArgs &a, hipStream_t s) {
    if (P == 16 && N == 16) return launch_gdn_wide_pn<16, 16>(st, a, s);
    if (P == 64 && N == 64) return launch_gdn_wide_pn<64, 64>(st, a, s);
    if (P == 64 && N == 128) return launch_gdn_wide_pn<64, 128>(st, a, s);
    if (P == 128 && N == 128) return launch_gdn_wide_pn<128, 128>(st, a, s);
    return hipErrorInvalidValue;
}

// W = 1: the register kernel; windows of 2 and more: the matrix cores (the
// register kernel's per-row sums for several positions took 68 to 256
// registers and measured 175 / 518 us at W = 4 / 8 with a float32
// checkpoint, 426 / 867 us with an e4m3 copy, against 218 - 243 us for the
// matrix cores at W = 9 .. 16; B=256, H=32, P=N=128)
hipError_t launch_gdn_verify(int P, int N, int st, const DecodeArgs &a, hipStream_t s) {
    if (a.W < 1 || a.W > kMaxWideWindow || a.W > a.r.L) return hipErrorInvalidValue;
    if (a.W > 1) return launch_gdn_wide(P, N, st, a, s);
    if (P == 16 && N == 16) return launch_gdn_decode_pn<16, 16>(st, a, s);
    if (P == 64 && N == 64) return launch_gdn_decode_pn<64, 64>(st, a, s);
    if (P == 64 && N == 128) return launch_gdn_decode_pn<64, 128>(st, a, s);
    if (P == 128 && N == 128) return launch_gdn_decode_pn<128, 128>(st, a, s);
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Fold (flush) and the eager step


// Thread layout of the fold: LPRW lanes share a row (8, or 4 for 16-column
// rows), lane j of a row holding its 16-byte pieces j, j + LPRW, ..., so that
// one load instruction covers LPRW consecutive pieces of every row it
// touches: whole 128-byte lines.  A lane holds RPL rows.
template <int P, int N>
struct GdnFoldShape {
    static constexpr int LPRW = N / 4 < 8 ? N / 4 : 8;      // lanes a row
    static constexpr int PPL = N / 4 / LPRW;                // 16-byte pieces of a row a lane holds
    static constexpr int LR = P * LPRW;                     // lane-rows of the tile
    static constexpr int NT = LR < 256 ? LR : 256;
    static constexpr int RPL = LR / NT;                     // rows a lane holds
    static constexpr int RSTEP = NT / LPRW;                 // rows between a lane's rows
    static_assert(LR % NT == 0 && NT % 64 == 0 && N % (4 * LPRW) == 0, "fold tiling");
};

// SIN: the state read -- the float32 checkpoint, or (the copy being the only
// checkpoint) a bf16 / e4m3 / MX FP4 copy, widened exactly and scaled.
// COPY: the copy written from the folded state (-1: none), with the same
// quantisers as the Mamba-2 flush: bf16 nearest even; e4m3 with one scale
// per head = amax / 448 and a correctly rounded division; MX FP4 blocks of
// 32 values (8 neighbouring lanes) with E8M0 scales.  WMASTER: the float32
// checkpoint is written.  A shared copy is rewritten in place: every lane
// reads its own codes (and its block's scale) before the fold and writes
// them after, and the e4m3 scale is written after the workgroup's barrier.
template <int P, int N, bool IOB, bool EMIT, int SIN = ST_F32, int COPY = -1, bool WMASTER = true>
__global__ __launch_bounds__((GdnFoldShape<P, N>::NT)) void gdn_fold_kernel(GdnFoldArgs args) {
    using FS = GdnFoldShape<P, N>;
    constexpr int LPRW = FS::LPRW, PPL = FS::PPL, NT = FS::NT, RPL = FS::RPL, RSTEP = FS::RSTEP;
    constexpr int LM = EMIT ? 1 : kMaxRing;
    constexpr int RBITS = __builtin_ctz(LPRW);
    static_assert(!EMIT || (SIN == ST_F32 && COPY < 0 && WMASTER), "the eager step reads and writes float32");
    __shared__ __align__(16) float s_k[LM][N];
    __shared__ float s_v[LM][P];
    __shared__ float s_ab[2][LM];   // alpha_m, beta_m
    __shared__ __align__(16) float s_q[EMIT ? N : 4];   // eager: the token's query
    __shared__ float s_red[COPY == ST_FP8 ? NT / 64 : 1];

    const RingView &r = args.r;
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int H = r.H;
    const int b = lid / H, h = lid % H;
    const int g = (h * r.G) / H;
    const int tid = threadIdx.x;
    const int row0 = tid / LPRW, jp = tid % LPRW;   // first row, piece offset within a row
    const size_t bh = (size_t)b * H + h;
    const size_t tile = bh * (size_t)(P * N);

    // (base is read once: after this workgroup's arrival the sequence's last
    // workgroup may move it)
    int count = 1, pos = 0, base = 0;
    if constexpr (!EMIT) {
        base = r.base[b];
        pos = r.pos[b];
        count = pos - base;
        if (count < (args.min_count > 1 ? args.min_count : 1)) return;   // uniform: nothing to fold
    }
    // every wavefront of a fold arrives at its group's counter right after
    // its own pointer read (one arrival per wavefront)
    int prev = -1;
    if constexpr (!EMIT) {
        if ((tid & 63) == 0) prev = atomicAdd(&args.sync[((size_t)b * (r.G + 1) + g) * kSyncStride], 1);
    }

    // this lane's pieces of its rows (element offsets within the head's tile)
    auto piece = [&](int i, int u) -> size_t { return (size_t)(row0 + RSTEP * i) * N + 4 * (jp + LPRW * u); };
    f32x4 s[RPL][PPL];
    if constexpr (SIN == ST_F32) {
#pragma unroll
        for (int i = 0; i < RPL; ++i)
#pragma unroll
            for (int u = 0; u < PPL; ++u)
                s[i][u] = __builtin_nontemporal_load(
                    reinterpret_cast<const f32x4 *>(static_cast<const float *>(args.S_in) + tile + piece(i, u)));
    } else if constexpr (SIN == ST_BF16) {
#pragma unroll
        for (int i = 0; i < RPL; ++i)
#pragma unroll
            for (int u = 0; u < PPL; ++u) {
                const u32x2 w = *reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(args.S_in) + tile + piece(i, u));
                s[i][u] = f32x4{bf16_bits_to_f32(w.x & 0xffffu), bf16_bits_to_f32(w.x >> 16),
                                bf16_bits_to_f32(w.y & 0xffffu), bf16_bits_to_f32(w.y >> 16)};
            }
    } else if constexpr (SIN == ST_FP8) {
        const float sc = static_cast<const float *>(args.scale_in)[bh];
#pragma unroll
        for (int i = 0; i < RPL; ++i)
#pragma unroll
            for (int u = 0; u < PPL; ++u) {
                float x[4];
                fp8x4_to_f32(*reinterpret_cast<const uint32_t *>(static_cast<const uint8_t *>(args.S_in) + tile + piece(i, u)), x);
                s[i][u] = f32x4{x[0] * sc, x[1] * sc, x[2] * sc, x[3] * sc};
            }
    } else {
        static_assert(SIN == ST_FP4, "state kind");
#pragma unroll
        for (int i = 0; i < RPL; ++i)
#pragma unroll
            for (int u = 0; u < PPL; ++u) {
                const size_t e0 = tile + piece(i, u);
                const uint32_t w = *reinterpret_cast<const uint16_t *>(static_cast<const uint8_t *>(args.S_in) + e0 / 2);
                const int se = (int)static_cast<const uint8_t *>(args.scale_in)[e0 / 32] - 127;
                float x[4];
                fp4_pair_to_f32(w, 0, x);
                fp4_pair_to_f32(w, 1, x + 2);
                s[i][u] = f32x4{ldexpf(x[0], se), ldexpf(x[1], se), ldexpf(x[2], se), ldexpf(x[3], se)};   // exact
            }
    }
    // the entries: k rows, v rows, alpha and beta, staged in LDS
    auto ld = [&](const void *base_ptr, size_t i) -> float {
        if constexpr (IOB) return bf16_bits_to_f32(static_cast<const uint16_t *>(base_ptr)[i]);
        else return static_cast<const float *>(base_ptr)[i];
    };
    if constexpr (EMIT) {
        for (int i = tid; i < N; i += NT) s_k[0][i] = ld(args.k, ((size_t)b * r.G + g) * N + i);
        for (int i = tid; i < P; i += NT) s_v[0][i] = ld(args.v, bh * P + i);
        for (int i = tid; i < N; i += NT) s_q[i] = ld(args.q, ((size_t)b * r.G + g) * N + i);
        if (tid == 0) {
            s_ab[0][0] = args.alpha[bh];
            s_ab[1][0] = args.beta[bh];
        }
    } else {
        const int L = r.L;
        const int bmod = base % L;
        const size_t gring = ((size_t)b * r.G + g) * L, hring = bh * L;
        gdn_stage_rows<LM, N, NT, IOB>(r.k, gring, bmod, L, count, tid, s_k);
        gdn_stage_rows<LM, P, NT, IOB>(r.v, hring, bmod, L, count, tid, s_v);
        if (tid < count) {
            s_ab[0][tid] = r.a[dta_index(b, bh, H, L, ring_slot(bmod, tid, L))];
            s_ab[1][tid] = r.dt[dta_index(b, bh, H, L, ring_slot(bmod, tid, L))];
        }
    }
    __syncthreads();

    // entry after entry, every row: s <- alpha (s - beta (s . k) k) + beta v_p k
    //                                   = alpha s + beta (v_p - alpha (s . k)) k
    for (int m = 0; m < count; ++m) {
        const float am = s_ab[0][m], bm = s_ab[1][m];
        f32x4 kk[PPL];
#pragma unroll
        for (int u = 0; u < PPL; ++u) kk[u] = *reinterpret_cast<const f32x4 *>(&s_k[m][4 * (jp + LPRW * u)]);
        float d[RPL];
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int u = 0; u < PPL; ++u)
                acc = fmaf(s[i][u].x, kk[u].x, fmaf(s[i][u].y, kk[u].y, fmaf(s[i][u].z, kk[u].z, fmaf(s[i][u].w, kk[u].w, acc))));
            d[i] = acc;
        }
#pragma unroll
        for (int bit = RBITS - 1; bit >= 0; --bit)
#pragma unroll
            for (int i = 0; i < RPL; ++i) d[i] += lane_partner(d[i], bit);   // the row's other pieces
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const float c = bm * s_v[m][row0 + RSTEP * i] - bm * am * d[i];
#pragma unroll
            for (int u = 0; u < PPL; ++u) {
                s[i][u].x = fmaf(c, kk[u].x, am * s[i][u].x);
                s[i][u].y = fmaf(c, kk[u].y, am * s[i][u].y);
                s[i][u].z = fmaf(c, kk[u].z, am * s[i][u].z);
                s[i][u].w = fmaf(c, kk[u].w, am * s[i][u].w);
            }
        }
    }
    if constexpr (WMASTER) {
#pragma unroll
        for (int i = 0; i < RPL; ++i)
#pragma unroll
            for (int u = 0; u < PPL; ++u)
                __builtin_nontemporal_store(s[i][u], reinterpret_cast<f32x4 *>(args.S_out + tile + piece(i, u)));
    }
    if constexpr (COPY == ST_BF16) {
        uint16_t *cp = static_cast<uint16_t *>(args.copy_out) + tile;
#pragma unroll
        for (int i = 0; i < RPL; ++i)
#pragma unroll
            for (int u = 0; u < PPL; ++u) {
                u32x2 o;
                o.x = f32x2_to_bf16_pair(s[i][u].x, s[i][u].y);
                o.y = f32x2_to_bf16_pair(s[i][u].z, s[i][u].w);
                *reinterpret_cast<u32x2 *>(cp + piece(i, u)) = o;
            }
    } else if constexpr (COPY == ST_FP8) {
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < RPL; ++i)
#pragma unroll
            for (int u = 0; u < PPL; ++u)
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(s[i][u].x), fabsf(s[i][u].y)), fmaxf(fabsf(s[i][u].z), fabsf(s[i][u].w))));
#pragma unroll
        for (int bit = 5; bit >= 0; --bit) amax = fmaxf(amax, lane_partner(amax, bit));
        if ((tid & 63) == 0) s_red[tid / 64] = amax;
        __syncthreads();
        amax = s_red[0];
#pragma unroll
        for (int i = 1; i < NT / 64; ++i) amax = fmaxf(amax, s_red[i]);
        const float sig = amax > 0.f ? amax / 448.0f : 1.0f;   // correctly rounded divide
        const ScaleDiv dv(sig);
        uint8_t *cp = static_cast<uint8_t *>(args.copy_out) + tile;
        dv.run([&](auto div) {
#pragma unroll
            for (int i = 0; i < RPL; ++i)
#pragma unroll
                for (int u = 0; u < PPL; ++u)
                    *reinterpret_cast<uint32_t *>(cp + piece(i, u)) =
                        f32x4_to_fp8(div(s[i][u].x), div(s[i][u].y), div(s[i][u].z), div(s[i][u].w));
        });
        if (tid == 0) static_cast<float *>(args.scale_out)[bh] = sig;
    } else if constexpr (COPY == ST_FP4) {
        // a block of 32 values is one piece of each of 8 neighbouring lanes
        // (of one row, or of two 16-value rows)
        uint8_t *cp = static_cast<uint8_t *>(args.copy_out);
        uint8_t *scl = static_cast<uint8_t *>(args.scale_out);
#pragma unroll
        for (int i = 0; i < RPL; ++i)
#pragma unroll
            for (int u = 0; u < PPL; ++u) {
                const f32x4 x = s[i][u];
                float amax = fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w)));
#pragma unroll
                for (int bit = 2; bit >= 0; --bit) amax = fmaxf(amax, lane_partner(amax, bit));
                const int se = mxfp4_block_exp(amax);
                const size_t e0 = tile + piece(i, u);
                *reinterpret_cast<uint16_t *>(cp + e0 / 2) = mxfp4_codes4(x.x, x.y, x.z, x.w, se);
                if ((tid & 7) == 0) scl[e0 / 32] = (uint8_t)(se + 127);
            }
    }
    if constexpr (EMIT) {
        // y_p = S_t[p] . q (the query from the call)
        f32x4 qq[PPL];
#pragma unroll
        for (int u = 0; u < PPL; ++u) qq[u] = *reinterpret_cast<const f32x4 *>(&s_q[4 * (jp + LPRW * u)]);
        float yq[RPL];
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int u = 0; u < PPL; ++u)
                acc = fmaf(s[i][u].x, qq[u].x, fmaf(s[i][u].y, qq[u].y, fmaf(s[i][u].z, qq[u].z, fmaf(s[i][u].w, qq[u].w, acc))));
            yq[i] = acc;
        }
#pragma unroll
        for (int bit = RBITS - 1; bit >= 0; --bit)
#pragma unroll
            for (int i = 0; i < RPL; ++i) yq[i] += lane_partner(yq[i], bit);
        if (jp == 0) {
#pragma unroll
            for (int i = 0; i < RPL; ++i) args.y[bh * P + row0 + RSTEP * i] = yq[i];
        }
    } else {
        // last wavefront of its group: the group arrives at the sequence's
        // counter; the last group means every wavefront has read base
        if ((tid & 63) == 0 && prev == r.H / r.G * (NT / 64) - 1) {
            int32_t *seq = args.sync + (size_t)b * (r.G + 1) * kSyncStride;
            atomicExch(seq + (size_t)g * kSyncStride, 0);
            if (atomicAdd(seq + (size_t)r.G * kSyncStride, 1) == r.G - 1) {
                atomicExch(seq + (size_t)r.G * kSyncStride, 0);
                args.base_out[b] = pos;
            }
        }
    }
}

template <int P, int N, bool EMIT, int SIN = ST_F32, int COPY = -1, bool WMASTER = true>
static hipError_t launch_gdn_fold_pn(const GdnFoldArgs &a, hipStream_t s) {
    const unsigned blocks = (unsigned)((size_t)a.r.B * a.r.H);
    if (a.r.io_bf16)
        gdn_fold_kernel<P, N, true, EMIT, SIN, COPY, WMASTER><<<blocks, GdnFoldShape<P, N>::NT, 0, s>>>(a);
    else
        gdn_fold_kernel<P, N, false, EMIT, SIN, COPY, WMASTER><<<blocks, GdnFoldShape<P, N>::NT, 0, s>>>(a);
    return hipGetLastError();
}

// the fold's configurations: float32 only; separated (float32 in, float32
// and a copy out); shared (a copy in, the same copy out)
template <int P, int N>
static hipError_t launch_gdn_flush_pn(int st_in, int st_copy, bool wm, const GdnFoldArgs &a, hipStream_t s) {
    if (st_in == ST_F32 && wm) {
        switch (st_copy) {
            case -1: return launch_gdn_fold_pn<P, N, false>(a, s);
            case ST_BF16: return launch_gdn_fold_pn<P, N, false, ST_F32, ST_BF16>(a, s);
            case ST_FP8: return launch_gdn_fold_pn<P, N, false, ST_F32, ST_FP8>(a, s);
            case ST_FP4: return launch_gdn_fold_pn<P, N, false, ST_F32, ST_FP4>(a, s);
            default: return hipErrorInvalidValue;
        }
    }
    if (!wm && st_in == st_copy) {
        switch (st_in) {
            case ST_BF16: return launch_gdn_fold_pn<P, N, false, ST_BF16, ST_BF16, false>(a, s);
            case ST_FP8: return launch_gdn_fold_pn<P, N, false, ST_FP8, ST_FP8, false>(a, s);
            case ST_FP4: return launch_gdn_fold_pn<P, N, false, ST_FP4, ST_FP4, false>(a, s);
            default: return hipErrorInvalidValue;
        }
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gdn_flush(int P, int N, int st_in, int st_copy, bool write_master, const GdnFoldArgs &a,
                            hipStream_t s) {
    if (a.r.L > kMaxRing || !a.sync || !a.base_out) return hipErrorInvalidValue;
    if (P == 16 && N == 16) return launch_gdn_flush_pn<16, 16>(st_in, st_copy, write_master, a, s);
    if (P == 64 && N == 64) return launch_gdn_flush_pn<64, 64>(st_in, st_copy, write_master, a, s);
    if (P == 64 && N == 128) return launch_gdn_flush_pn<64, 128>(st_in, st_copy, write_master, a, s);
    if (P == 128 && N == 128) return launch_gdn_flush_pn<128, 128>(st_in, st_copy, write_master, a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_gdn_eager(int P, int N, const GdnFoldArgs &a, hipStream_t s) {
    if (P == 16 && N == 16) return launch_gdn_fold_pn<16, 16, true>(a, s);
    if (P == 64 && N == 64) return launch_gdn_fold_pn<64, 64, true>(a, s);
    if (P == 64 && N == 128) return launch_gdn_fold_pn<64, 128, true>(a, s);
    if (P == 128 && N == 128) return launch_gdn_fold_pn<128, 128, true>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace replay
