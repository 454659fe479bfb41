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

namespace replay {

// ---------------------------------------------------------------------------
// Output-only route: decode (W = 1) and verify (W <= kMaxWindow)

// PR of the head's P rows per workgroup: a 128 x 128 head is streamed by two
// workgroups of 64 rows (4 + 1 wavefronts each; six fit a compute unit where
// three of 8 + 1 did), each running the whole chain for its own rows.
template <int P, int N, int WM, int LM, bool IOB, int PR = P>
struct GdnShape {
    using Sh = DecodeShape<PR, N, ST_F32, WM>;
    static constexpr int SPL = P / PR;            // workgroups a head
    static constexpr int NTS = Sh::NTS;           // streaming threads
    static constexpr int NT = NTS + 64;           // + the chain wavefront
    static constexpr int E = (N + 63) / 64;       // w elements a chain lane holds (n = lane + 64 e)
    static constexpr int VR = (PR + 63) / 64;     // outputs a chain lane accumulates (p = lane + 64 r)
    static_assert(P % PR == 0, "whole row blocks");
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
// entry t_w = count - W + w.  Writes s_w0[w][n] = w_0 of position w and, for
// the PR rows p0 .. p0 + PR, s_r[w][p - p0] = sum_{j<=t_w} beta_j (k_j . w_j) v_j[p].
template <int P, int N, int WM, int LM, bool IOB, int PR>
__device__ __forceinline__ void gdn_chain_wave(const RingView &r, int lane, int b, int g, size_t bh, int base,
                                               int count, int W, int p0, float (*s_k)[N], float (*s_v)[PR],
                                               float (*s_w0)[N], float (*s_r)[PR]) {
    using GS = GdnShape<P, N, WM, LM, IOB, PR>;
    constexpr int E = GS::E, VR = GS::VR;
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
        const int t = count - W + (w < W ? w : W - 1);
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
    gdn_stage_rows<LM, N, 64, IOB>(r.k, gring, bmod, L, count, lane, s_k);
    gdn_stage_rows<LM, PR, 64, IOB, P>(r.v, hring, bmod, L, count, lane, s_v, p0);
    wave_lds_sync();   // every lane's k and v rows are in LDS

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
                if (w < W && m <= count - W + w) {   // uniform
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
        if (w < W) {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (lane + 64 * e < N) s_w0[w][lane + 64 * e] = wv[w][e];
#pragma unroll
            for (int rr = 0; rr < VR; ++rr)
                if (lane + 64 * rr < PR) s_r[w][lane + 64 * rr] = acc[w][rr];
        }
    }
}

template <int P, int N, int WM, int LM, bool IOB, int PR>
__global__ __launch_bounds__((GdnShape<P, N, WM, LM, IOB, PR>::NT)) void gdn_verify_kernel(DecodeArgs args) {
    using GS = GdnShape<P, N, WM, LM, IOB, PR>;
    using Sh = typename GS::Sh;
    constexpr int VEC = Sh::VEC, NTS = Sh::NTS, ITER = Sh::ITER, LPR = Sh::LPR, RPI = Sh::RPI;
    using RR = RowReduce<ITER, LPR>;
    static_assert(VEC == 4, "float32 chunks");

    __shared__ __align__(16) float s_k[LM][N];
    __shared__ __align__(16) float s_v[LM][PR];
    __shared__ __align__(16) float s_w0[WM][N];
    __shared__ float s_r[WM][PR];

    const RingView &r = args.r;
    const int W = args.W;
    // consecutive workgroups: the row blocks of a head, then the heads of a
    // group (same compute die, whose L2 holds the group's k rows)
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int H = r.H;
    const int hb = lid / GS::SPL, p0 = (lid % GS::SPL) * PR;
    const int b = hb / H, h = hb % H;
    const int g = (h * r.G) / H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t bh = (size_t)b * H + h;
    const size_t tile = bh * (size_t)(P * N) + (size_t)p0 * N;

    const int base = r.base[b];
    const int pos = r.pos[b];
    const int count = pos - base;
    Chunk<ST_F32, VEC> ch[ITER];
    if (wave < NTS / 64) {
#pragma unroll
        for (int i = 0; i < ITER; ++i) ch[i].load(args.S, tile + (size_t)(i * NTS + tid) * VEC);
    }
    if (count < W) {   // uniform over the workgroup
        for (int i = tid; i < W * PR; i += GS::NT)
            args.y[(((size_t)b * W + i / PR) * H + h) * P + p0 + i % PR] = __builtin_nanf("");
        if (tid == 0) raise_seq_error(r.err, b, REPLAY_SEQERR_TOO_FEW);
        return;
    }
    if (wave == NTS / 64)
        gdn_chain_wave<P, N, WM, LM, IOB, PR>(r, lane, b, g, bh, base, count, W, p0, s_k, s_v, s_w0, s_r);
    __syncthreads();
    if (wave == NTS / 64) return;

    // S0 w_0 for every position: partial sums over this lane's chunks, then
    // the row reduction across the LPR lanes of a row
    const int col0 = (tid % LPR) * VEC;
    float part[ITER][WM];
#pragma unroll
    for (int w = 0; w < WM; ++w) {
        f32x4 q = {0.f, 0.f, 0.f, 0.f};
        if (w < W) q = *reinterpret_cast<const f32x4 *>(&s_w0[w][col0]);
#pragma unroll
        for (int i = 0; i < ITER; ++i) {
            const f32x4 x = ch[i].raw;
            part[i][w] = fmaf(x.x, q.x, fmaf(x.y, q.y, fmaf(x.z, q.z, x.w * q.w)));
        }
    }
    RR::template run<WM>(part, lane);
    if (RR::writer(lane)) {
        const int hi = RR::halving_index(lane);
#pragma unroll
        for (int e = 0; e < RR::FINAL; ++e) {
            const int p = (e + RR::FINAL * hi) * RPI + tid / LPR;
#pragma unroll
            for (int w = 0; w < WM; ++w)
                if (w < W) args.y[(((size_t)b * W + w) * H + h) * P + p0 + p] = part[e][w] + s_r[w][p];
        }
    }
}

template <int P, int N, int WM, int LM>
static hipError_t launch_gdn_verify_lm(const DecodeArgs &a, hipStream_t s) {
    constexpr int PR = P == 128 ? 64 : P;
    const unsigned blocks = (unsigned)((size_t)a.r.B * a.r.H * (P / PR));
    if (a.r.io_bf16)
        gdn_verify_kernel<P, N, WM, LM, true, PR><<<blocks, GdnShape<P, N, WM, LM, true, PR>::NT, 0, s>>>(a);
    else
        gdn_verify_kernel<P, N, WM, LM, false, PR><<<blocks, GdnShape<P, N, WM, LM, false, PR>::NT, 0, s>>>(a);
    return hipGetLastError();
}

template <int P, int N, int WM>
static hipError_t launch_gdn_verify_w(const DecodeArgs &a, hipStream_t s) {
    if (a.r.L <= 16) return launch_gdn_verify_lm<P, N, WM, 16>(a, s);
    return launch_gdn_verify_lm<P, N, WM, kMaxRing>(a, s);
}

template <int P, int N>
static hipError_t launch_gdn_verify_pn(const DecodeArgs &a, hipStream_t s) {
    if (a.W == 1) return launch_gdn_verify_w<P, N, 1>(a, s);
    if (a.W <= 4) return launch_gdn_verify_w<P, N, 4>(a, s);
    return launch_gdn_verify_w<P, N, kMaxWindow>(a, s);
}

hipError_t launch_gdn_verify(int P, int N, const DecodeArgs &a, hipStream_t s) {
    if (a.W < 1 || a.W > kMaxWindow || a.W > a.r.L) return hipErrorInvalidValue;
    if (P == 16 && N == 16) return launch_gdn_verify_pn<16, 16>(a, s);
    if (P == 64 && N == 64) return launch_gdn_verify_pn<64, 64>(a, s);
    if (P == 64 && N == 128) return launch_gdn_verify_pn<64, 128>(a, s);
    if (P == 128 && N == 128) return launch_gdn_verify_pn<128, 128>(a, s);
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

template <int P, int N, bool IOB, bool EMIT>
__global__ __launch_bounds__((GdnFoldShape<P, N>::NT)) void gdn_fold_kernel(GdnFoldArgs args) {
    using FS = GdnFoldShape<P, N>;
    constexpr int LPRW = FS::LPRW, PPL = FS::PPL, NT = FS::NT, RPL = FS::RPL, RSTEP = FS::RSTEP;
    constexpr int LM = EMIT ? 1 : kMaxRing;
    constexpr int RBITS = __builtin_ctz(LPRW);
    __shared__ __align__(16) float s_k[LM][N];
    __shared__ float s_v[LM][P];
    __shared__ float s_ab[2][LM];   // alpha_m, beta_m
    __shared__ __align__(16) float s_q[EMIT ? N : 4];   // eager: the token's query

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
    int prev = -1;
    if constexpr (!EMIT) {
        if (tid == 0) prev = atomicAdd(&args.sync[((size_t)b * (r.G + 1) + g) * kSyncStride], 1);
    }

    // this lane's pieces of its rows
    f32x4 s[RPL][PPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i)
#pragma unroll
        for (int u = 0; u < PPL; ++u)
            s[i][u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(
                args.S_in + tile + (size_t)(row0 + RSTEP * i) * N + 4 * (jp + LPRW * u)));
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
#pragma unroll
    for (int i = 0; i < RPL; ++i)
#pragma unroll
        for (int u = 0; u < PPL; ++u)
            __builtin_nontemporal_store(s[i][u], reinterpret_cast<f32x4 *>(
                args.S_out + tile + (size_t)(row0 + RSTEP * i) * N + 4 * (jp + LPRW * u)));
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
        // last workgroup of its group: the group arrives at the sequence's
        // counter; the last group means every workgroup has read base
        if (tid == 0 && prev == r.H / r.G - 1) {
            int32_t *seq = args.sync + (size_t)b * (r.G + 1) * kSyncStride;
            atomicExch(seq + (size_t)g * kSyncStride, 0);
            if (atomicAdd(seq + (size_t)r.G * kSyncStride, 1) == r.G - 1) {
                atomicExch(seq + (size_t)r.G * kSyncStride, 0);
                args.base_out[b] = pos;
            }
        }
    }
}

template <int P, int N, bool EMIT>
static hipError_t launch_gdn_fold_pn(const GdnFoldArgs &a, hipStream_t s) {
    const unsigned blocks = (unsigned)((size_t)a.r.B * a.r.H);
    if (a.r.io_bf16)
        gdn_fold_kernel<P, N, true, EMIT><<<blocks, GdnFoldShape<P, N>::NT, 0, s>>>(a);
    else
        gdn_fold_kernel<P, N, false, EMIT><<<blocks, GdnFoldShape<P, N>::NT, 0, s>>>(a);
    return hipGetLastError();
}

template <bool EMIT>
static hipError_t launch_gdn_fold_any(int P, int N, const GdnFoldArgs &a, hipStream_t s) {
    if (P == 16 && N == 16) return launch_gdn_fold_pn<16, 16, EMIT>(a, s);
    if (P == 64 && N == 64) return launch_gdn_fold_pn<64, 64, EMIT>(a, s);
    if (P == 64 && N == 128) return launch_gdn_fold_pn<64, 128, EMIT>(a, s);
    if (P == 128 && N == 128) return launch_gdn_fold_pn<128, 128, EMIT>(a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_gdn_flush(int P, int N, const GdnFoldArgs &a, hipStream_t s) {
    if (a.r.L > kMaxRing || !a.sync || !a.base_out) return hipErrorInvalidValue;
    return launch_gdn_fold_any<false>(P, N, a, s);
}

hipError_t launch_gdn_eager(int P, int N, const GdnFoldArgs &a, hipStream_t s) {
    return launch_gdn_fold_any<true>(P, N, a, s);
}

}  // namespace replay
