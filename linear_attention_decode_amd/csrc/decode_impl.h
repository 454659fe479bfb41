// decode_impl.h -- output-only decode and speculative verify for gfx950.
//
// Computes, for the W newest ring entries t_w = count-W+1+w of every
// (sequence, head),
//     y_w = abar_{t_w} (S0 q_{t_w}) + sum_{j<=t_w} s_{j,t_w} v_j (k_j . q_{t_w})
// (page "ReplaySSM: Cachear Inputs, No Estado", section "Los dos caminos",
// eq. "Ruta solo salida"; "Paralelismo": every window position reads the
// same checkpoint and buffer, entry j is visible to position t when j <= t),
// with abar_t = prod_{m<=t} a_m and s_{j,t} = dt_j prod_{j<m<=t} a_m.
// Decode is W = 1.  The checkpoint (or its bf16 / e4m3 copy) is read once
// per call and never written.
//
// One workgroup per (sequence, head).  The head's P x N tile streams through
// registers in coalesced 16-byte chunks (the whole workgroup covers NT*16
// contiguous bytes per iteration), all chunk loads are issued before any
// other work so they overlap the ring arithmetic.  k_j . q is formed per
// group by the workgroup itself from the group's k ring (L2-resident: the
// XCD-aware block order keeps a group's heads on one XCD); with bf16 io the
// ring wavefront forms the dots and the ring term on the matrix cores.  Row
// sums are finished with a transposed halving reduction across the lanes of a
// row.
#pragma once
#include "ring_mx.h"

namespace replay {

// NARROW: 8-element chunks for the low-precision tiles of several heads per
// workgroup with float32 io (the register budget goes to the extra chunks in
// flight and to the widened queries).  With bf16 io the queries stay bf16
// pairs, so full 16-byte chunks fit.
template <int P, int N, int ST, int WM, bool NARROW = false>
struct DecodeShape {
    static constexpr int base_vec = ST == ST_F32 ? 4
                                  : (ST == ST_BF16 ? 8 : (NARROW ? 8 : (ST == ST_FP8 ? (WM == 1 ? 16 : 8) : (WM == 1 ? 32 : 8))));
    // at least one full wavefront of chunks per head
    static constexpr int VEC = (P * N / base_vec >= 64) ? base_vec
                             : ((P * N / (base_vec / 2) >= 64) ? base_vec / 2
                             : ((P * N / (base_vec / 4) >= 64) ? base_vec / 4 : base_vec / 8));
    static constexpr int CHUNKS = P * N / VEC;
    // streaming threads: at most 8 chunks a lane (4096 chunks: 8 wavefronts)
    static constexpr int NTS = CHUNKS >= 4096 ? 512 : (CHUNKS < 256 ? CHUNKS : 256);
    static constexpr int ITER = CHUNKS / NTS;
    // Lanes per state row: N / VEC, except for a float32 tile scored for a
    // window of WM >= 2 queries.  There 8 lanes share a row and lane jp holds
    // the row's 16-byte pieces jp, jp + 8, ... (PPL of them): a load
    // instruction still reads whole 128-byte lines (of 8 rows), a lane adds
    // its pieces of a row before any lane exchange, and each query's row
    // reduction takes 3 lane steps (DPP only) in place of 5.
    static constexpr int LPR = (ST == ST_F32 && WM >= 2 && N / VEC > 8) ? 8 : N / VEC;
    static constexpr int PPL = N / VEC / LPR;   // pieces of one row a lane holds
    static constexpr int RPL = ITER / PPL;      // rows a lane holds
    static constexpr int RPI = NTS / LPR;       // rows between a lane's rows
    static_assert(VEC >= 4, "chunk too small");
    static_assert(CHUNKS % NTS == 0 && NTS % 64 == 0, "bad tiling");
    static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "row group must sit in a wavefront");
    static_assert(ITER % PPL == 0, "a lane holds whole rows");
    // Element offset within the tile of chunk i of streaming thread tid: row
    // (i / PPL) * RPI + tid / LPR, piece tid % LPR + LPR * (i % PPL).  With
    // PPL = 1 this is (i * NTS + tid) * VEC: NTS contiguous chunks per i.
    static __device__ __forceinline__ int offset(int i, int tid) {
        return ((i / PPL) * RPI + tid / LPR) * N + VEC * (tid % LPR + LPR * (i % PPL));
    }
};

// The ring wavefront's work for one (sequence, head): group dots, segment
// weights and the ring term, all in registers; results go to LDS.
//   s_r[w][p] = sum_{j<=t_w} s_{j,t_w} (k_j . q_{t_w}) v_j[p],   s_abar[w] = abar_{t_w}
template <int P, int N, int WM, int LM, bool IOB>
__device__ __forceinline__ void ring_wave(const RingView &r, int lane, int b, int g, size_t bh, int base,
                                          int count, float (*s_r)[P], float *s_abar) {
    constexpr int W = WM;
    constexpr int TS = N / 8;               // lanes per k.q dot (8 elements each)
    constexpr int RPW = 64 / TS;            // ring entries per k instruction
    constexpr int KI = (LM + RPW - 1) / RPW;
    constexpr int VR = (P + 63) / 64;       // state rows per lane in the ring term
    static_assert(TS >= 1 && 64 % TS == 0, "dot teams");
    const int L = r.L;
    const size_t gring = ((size_t)b * r.G + g) * L;
    const size_t hring = bh * L;
    const int t0 = count - W;               // window position w is entry t0 + w (0-based)
    const int bmod = base % L;
    auto slot = [&](int j) { return ring_slot(bmod, j, L); };

    // every load first, from valid entries only (indices clamped to the live
    // range; values of clamped lanes are masked out below, never used)
    const int last = count - 1;
    float aj, dtj;
    {
        const int sl = slot(lane < count ? lane : last);
        aj = r.a[dta_index(b, bh, r.H, L, sl)];
        dtj = r.dt[dta_index(b, bh, r.H, L, sl)];
    }
    const int tl = lane % TS, te = lane / TS;
    IoVec<IOB, 8> kraw[KI];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
        const int j = i * RPW + te;
        kraw[i].load(r.k, (gring + slot(j < count ? j : last)) * N + tl * 8);
    }
    IoVec<IOB, 8> qraw[WM];
#pragma unroll
    for (int w = 0; w < WM; ++w) qraw[w].load(r.q, (gring + slot(t0 + (w < W ? w : W - 1))) * N + tl * 8);
    IoVec<IOB, 1> vraw[VR][LM];
#pragma unroll
    for (int rr = 0; rr < VR; ++rr)
#pragma unroll
        for (int j = 0; j < LM; ++j) {
            const int p = lane + 64 * rr;
            vraw[rr][j].load(r.v, (hring + slot(j < count ? j : last)) * P + (p < P ? p : P - 1));
        }
    if (lane >= count) {
        aj = 1.f;
        dtj = 0.f;
    }

    // dots c[w][j], then moved so that lane j holds c[w][j]
    float cw[WM];
#pragma unroll
    for (int w = 0; w < WM; ++w) cw[w] = 0.f;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
#pragma unroll
        for (int w = 0; w < WM; ++w) {
            if (w < W) {
                float d = dot8(kraw[i], qraw[w]);
                d = group_sum<TS>(d);
                const float moved = __shfl(d, (lane % RPW) * TS);
                if (lane / RPW == i) cw[w] = moved;
            }
        }
    }

    // segment weights, left to right: s_{j,t} = dt_j a_{j+1} ... a_t, abar_t = a_0 ... a_t
    float sw[WM], ab[WM];
    float prod = dtj, run = 1.f;
#pragma unroll
    for (int w = 0; w < WM; ++w) sw[w] = ab[w] = 0.f;
#pragma unroll
    for (int m = 0; m < LM; ++m) {
        if (m < count) {
            const float am = bcast(aj, m);
            if (m > lane) prod *= am;
            run *= am;
#pragma unroll
            for (int w = 0; w < WM; ++w)
                if (m == t0 + w) {
                    sw[w] = prod;
                    ab[w] = run;
                }
        }
    }
    float coef[WM];
#pragma unroll
    for (int w = 0; w < WM; ++w) coef[w] = (w < W && lane <= t0 + w) ? sw[w] * cw[w] : 0.f;

    // ring term, entries in order
    float acc[VR][WM];
#pragma unroll
    for (int rr = 0; rr < VR; ++rr)
#pragma unroll
        for (int w = 0; w < WM; ++w) acc[rr][w] = 0.f;
#pragma unroll
    for (int j = 0; j < LM; ++j) {
        if (j < count) {
#pragma unroll
            for (int w = 0; w < WM; ++w) {
                if (w < W && j <= t0 + w) {
                    const float cj = bcast(coef[w], j);
#pragma unroll
                    for (int rr = 0; rr < VR; ++rr) acc[rr][w] = fmaf(cj, vraw[rr][j].value(), acc[rr][w]);
                }
            }
        }
    }
#pragma unroll
    for (int rr = 0; rr < VR; ++rr) {
        const int p = lane + 64 * rr;
        if (p < P) {
#pragma unroll
            for (int w = 0; w < WM; ++w)
                if (w < W) s_r[w][p] = acc[rr][w];
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int w = 0; w < WM; ++w)
            if (w < W) s_abar[w] = ab[w];
    }
}

// The same work for bf16 io on the matrix cores (ring_mx.h), operands read
// from the ring: every entry and query from its ring slot, indices clamped to
// the live range.  This wavefront covers entries j0..j0+15.
template <int P, int N, int WM, int LM>
__device__ __forceinline__ void ring_wave_mx(const RingView &r, int lane, int j0, int b, int g, size_t bh,
                                             int base, int count, float (*s_r)[P], float *s_abar,
                                             float (*s_sw)[LM]) {
    using MX = MxRing<P, N, WM, LM>;
    const int L = r.L;
    const size_t gring = ((size_t)b * r.G + g) * L;
    const size_t hring = bh * L;
    const int t0 = count - WM;
    const int bmod = base % L;
    auto slot = [&](int j) { return ring_slot(bmod, j, L); };
    const int last = count - 1;
    const int lr = lane & 15, lq = lane >> 4;

    MX m;
    m.j0 = j0;
    {
        const int sl = slot(lane < count ? lane : last);
        m.aj = r.a[dta_index(b, bh, r.H, L, sl)];
        m.dtj = r.dt[dta_index(b, bh, r.H, L, sl)];
    }
#pragma unroll
    for (int kb = 0; kb < MX::KB; ++kb) {
        const int c = MX::col(kb, lane);
        const int j = j0 + lr;
        m.ka[kb] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(r.k) +
                                                    (gring + slot(j < count ? j : last)) * N + c);
        m.qb[kb] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(r.q) +
                                                    (gring + slot(t0 + (lr < WM ? lr : WM - 1))) * N + c);
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
    m.weights(lane, count, s_abar, s_sw);
    m.term(lane, dk, s_r, s_sw);
}

// Ring wavefronts of the decode kernel: two for a 32-entry ring with bf16 io
// (one per 16-entry block), else one.
template <int LM, bool IOB>
constexpr int ring_waves() { return IOB ? LM / 16 : 1; }

// Heads per workgroup: low-precision tiles are small, so one workgroup takes
// HPW heads of one group (their tiles are contiguous in memory and stream as
// one taller tile); each head keeps its own ring wavefront(s).  The per-
// workgroup latency of the ring work is then paid once per HPW heads.
// (Decode only: a verify window's extra queries and partial sums take the
// registers the extra chunks would need.)
template <int ST, int WM>
constexpr int heads_per_wg() { return (ST == ST_F32 || WM > 1) ? 1 : (ST == ST_BF16 ? 2 : 4); }

template <int P, int N, int ST, int WM, int LM, bool IOB, int HPW>
struct DecodeLaunch {
    using Sh = DecodeShape<P * HPW, N, ST, WM, (HPW > 1 && !IOB)>;
    static constexpr int NR = ring_waves<LM, IOB>();      // ring wavefronts per head
    static constexpr int NT = Sh::NTS + 64 * NR * HPW;
};

template <int P, int N, int ST, int WM, int LM, bool IOB, int HPW>
__global__ __launch_bounds__((DecodeLaunch<P, N, ST, WM, LM, IOB, HPW>::NT)) void decode_kernel(DecodeArgs args) {
    using DL = DecodeLaunch<P, N, ST, WM, LM, IOB, HPW>;
    using Sh = typename DL::Sh;
    constexpr int W = WM, PT = P * HPW;
    constexpr int VEC = Sh::VEC, NTS = Sh::NTS, ITER = Sh::ITER, LPR = Sh::LPR, RPI = Sh::RPI;
    constexpr int PPL = Sh::PPL, RPL = Sh::RPL;
    constexpr int NR = DL::NR, NT = DL::NT;
    using RR = RowReduce<RPL, LPR>;
    // float32 tile with several pieces of a row per lane: the window's
    // queries widened into LDS, one copy per streaming wavefront
    constexpr bool QLDS = ST == ST_F32 && PPL > 1;

    __shared__ float s_r[NR][HPW][WM][P];
    __shared__ float s_abar[HPW][WM];
    __shared__ __align__(16) float s_sw[HPW][IOB ? WM : 1][IOB ? LM : 4];
    __shared__ __align__(16) float s_qw[QLDS ? NTS / 64 : 1][QLDS ? WM : 1][QLDS ? N : 4];

    const RingView &r = args.r;
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int HW = r.H / HPW;
    const int b = lid / HW, h0 = (lid % HW) * HPW;
    const int g = (h0 * r.G) / r.H;   // the HPW heads share this group
    const int tid = threadIdx.x, lane = tid & 63;
    const int L = r.L, H = r.H;
    const size_t bh0 = (size_t)b * H + h0;

    // pointer pair first, then the state tiles (which do not depend on it)
    const int base = r.base[b];
    const int pos = r.pos[b];
    Chunk<ST, VEC> ch[ITER];
    const size_t tile = bh0 * (size_t)(P * N);
    if (tid < NTS) {
#pragma unroll
        for (int i = 0; i < ITER; ++i) {
            if constexpr (ST == ST_FP4)
                ch[i].load_mx(args.S, args.scale, tile + (size_t)Sh::offset(i, tid));
            else
                ch[i].load(args.S, tile + (size_t)Sh::offset(i, tid));
        }
    }
    const int count = pos - base;
    if (count < W) {  // uniform over the workgroup
        for (int i = tid; i < W * PT; i += NT) {
            const int w = i / PT, pp = i % PT;
            args.y[(((size_t)b * W + w) * H + h0) * P + pp] = __builtin_nanf("");
        }
        if (tid == 0) raise_seq_error(r.err, b, REPLAY_SEQERR_TOO_FEW);
        return;
    }

    float part[RPL][WM];
    if (tid < NTS) {
        // queries of the window positions at this lane's columns
        const int col0 = (tid % LPR) * VEC;
        const size_t gring = ((size_t)b * r.G + g) * L;
        const int bmod = base % L;
        if constexpr (IOB && ST != ST_F32) {
            // low-precision tile, bf16 queries: the queries stay bf16 pairs
            // and every chunk goes to bf16 pairs (exact for bf16, e4m3 and
            // E2M1 values), dotted by v_dot2_f32_bf16
            constexpr int QW = VEC / 2;   // words of bf16 pairs per query
            uint32_t qw[WM][QW];
#pragma unroll
            for (int w = 0; w < WM; ++w) {
                const uint32_t *row = reinterpret_cast<const uint32_t *>(
                    static_cast<const uint16_t *>(r.q) +
                    (gring + ring_slot(bmod, count - W + (w < W ? w : W - 1), L)) * N + col0);
                if constexpr (QW % 4 == 0) {
#pragma unroll
                    for (int e = 0; e < QW / 4; ++e) {
                        const uint4 u = reinterpret_cast<const uint4 *>(row)[e];
                        qw[w][4 * e] = u.x; qw[w][4 * e + 1] = u.y; qw[w][4 * e + 2] = u.z; qw[w][4 * e + 3] = u.w;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < QW; ++e) qw[w][e] = row[e];
                }
            }
#pragma unroll
            for (int i = 0; i < ITER; ++i) {
#pragma unroll
                for (int w = 0; w < WM; ++w) {
                    float acc = ch[i].dot_bf16(qw[w]);
                    if constexpr (ST == ST_FP4) acc = ldexpf(acc, ch[i].se);   // the block's scale, exact
                    part[i][w] = acc;
                }
            }
        } else if constexpr (QLDS) {
            // This wavefront widens the window's queries into its own LDS
            // rows (a wavefront-level exchange, no workgroup barrier), then
            // forms the row sums one query at a time from its pieces.
            float *sq = &s_qw[tid >> 6][0][0];
            constexpr int QP = WM * N / 4;   // 4-element pieces of the queries
#pragma unroll
            for (int k0 = 0; k0 < QP; k0 += 64) {
                const int k = k0 + lane;
                if (k < QP) {
                    const int w = k / (N / 4), c = 4 * (k % (N / 4));
                    IoVec<IOB, 4> t;
                    t.load(r.q, (gring + ring_slot(bmod, count - W + w, L)) * N + c);
                    float f[4];
                    t.widen(f);
                    *reinterpret_cast<f32x4 *>(sq + w * N + c) = f32x4{f[0], f[1], f[2], f[3]};
                }
            }
            wave_lds_sync();
            const int jp = tid % LPR;
#pragma unroll
            for (int w = 0; w < WM; ++w) {
                f32x4 qp[PPL];
#pragma unroll
                for (int u = 0; u < PPL; ++u) qp[u] = *reinterpret_cast<const f32x4 *>(sq + w * N + VEC * (jp + LPR * u));
#pragma unroll
                for (int rr = 0; rr < RPL; ++rr) {
                    f32x4 xp[PPL];
#pragma unroll
                    for (int u = 0; u < PPL; ++u) xp[u] = ch[rr * PPL + u].raw;
                    part[rr][w] = pieces_dot<PPL>(xp, qp);
                }
            }
        } else {
            IoVec<IOB, 4> qraw[WM][VEC / 4];
#pragma unroll
            for (int w = 0; w < WM; ++w) {
                const size_t off = (gring + ring_slot(bmod, count - W + (w < W ? w : W - 1), L)) * N + col0;
#pragma unroll
                for (int e = 0; e < VEC / 4; ++e) qraw[w][e].load(r.q, off + 4 * e);
            }
            float qv[WM][VEC];
#pragma unroll
            for (int w = 0; w < WM; ++w)
#pragma unroll
                for (int e = 0; e < VEC / 4; ++e) qraw[w][e].widen(&qv[w][4 * e]);
#pragma unroll
            for (int i = 0; i < ITER; ++i) {
                float x[VEC];
                ch[i].widen(x, 1.0f);
#pragma unroll
                for (int w = 0; w < WM; ++w) {
                    float acc = 0.f;
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc = fmaf(x[e], qv[w][e], acc);
                    if constexpr (ST == ST_FP4) acc = ldexpf(acc, ch[i].se);   // the block's scale, exact
                    part[i][w] = acc;
                }
            }
        }
        RR::template run<WM>(part, lane);
    } else {
        // ring wavefront: head hl, 16-entry block blk (wave-uniform, so the
        // buffer descriptors built from it stay in scalar registers)
        const int rwave = __builtin_amdgcn_readfirstlane((tid - NTS) >> 6);
        const int hl = rwave / NR, blk = rwave % NR;
        const size_t bh = bh0 + hl;
        if constexpr (IOB)
            ring_wave_mx<P, N, WM, LM>(r, lane, 16 * blk, b, g, bh, base, count, s_r[blk][hl], s_abar[hl], s_sw[hl]);
        else
            ring_wave<P, N, WM, LM, IOB>(r, lane, b, g, bh, base, count, s_r[0][hl], s_abar[hl]);
    }
    __syncthreads();

    if (tid < NTS && RR::writer(lane)) {
        const int hi = RR::halving_index(lane);
#pragma unroll
        for (int e = 0; e < RR::FINAL; ++e) {
            const int row = (e + RR::FINAL * hi) * RPI + tid / LPR;   // of the HPW stacked tiles
            const int hl = HPW == 1 ? 0 : row / P, p = HPW == 1 ? row : row % P;
            const float sc = (ST == ST_FP8) ? static_cast<const float *>(args.scale)[bh0 + hl] : 1.0f;
#pragma unroll
            for (int w = 0; w < WM; ++w) {
                if (w < W) {
                    float rt = s_r[0][hl][w][p];
                    if constexpr (NR == 2) rt += s_r[1][hl][w][p];   // block 0 + block 1
                    args.y[(((size_t)b * W + w) * H + h0) * P + row] = s_abar[hl][w] * (sc * part[e][w]) + rt;
                }
            }
        }
    }
}

template <int P, int N, int ST, int WM, int LM, bool IOB>
static hipError_t launch_one(const DecodeArgs &a, hipStream_t s) {
    constexpr int HPW = heads_per_wg<ST, WM>();
    // several heads per workgroup when they divide a group evenly
    if (HPW > 1 && (a.r.H / a.r.G) % HPW == 0) {
        using DL = DecodeLaunch<P, N, ST, WM, LM, IOB, HPW>;
        const unsigned blocks = (unsigned)((size_t)a.r.B * a.r.H / HPW);
        decode_kernel<P, N, ST, WM, LM, IOB, HPW><<<blocks, DL::NT, 0, s>>>(a);
    } else {
        using DL = DecodeLaunch<P, N, ST, WM, LM, IOB, 1>;
        const unsigned blocks = (unsigned)((size_t)a.r.B * a.r.H);
        decode_kernel<P, N, ST, WM, LM, IOB, 1><<<blocks, DL::NT, 0, s>>>(a);
    }
    return hipGetLastError();
}

template <int P, int N, int ST, int WM, bool IOB>
static hipError_t launch_l(const DecodeArgs &a, hipStream_t s) {
    if (a.r.L <= 16) return launch_one<P, N, ST, WM, 16, IOB>(a, s);
    return launch_one<P, N, ST, WM, kMaxRing, IOB>(a, s);
}

template <int P, int N, int ST, bool IOB>
static hipError_t launch_w(const DecodeArgs &a, hipStream_t s) {
    switch (a.W) {
        case 1: return launch_l<P, N, ST, 1, IOB>(a, s);
        case 2: return launch_l<P, N, ST, 2, IOB>(a, s);
        case 3: return launch_l<P, N, ST, 3, IOB>(a, s);
        case 4: return launch_l<P, N, ST, 4, IOB>(a, s);
        case 5: return launch_l<P, N, ST, 5, IOB>(a, s);
        case 6: return launch_l<P, N, ST, 6, IOB>(a, s);
        case 7: return launch_l<P, N, ST, 7, IOB>(a, s);
        case 8: return launch_l<P, N, ST, 8, IOB>(a, s);
        default: return hipErrorInvalidValue;
    }
}

template <int ST, bool IOB>
hipError_t launch_decode_st(int P, int N, const DecodeArgs &a, hipStream_t s) {
    if (P == 16 && N == 16) return launch_w<16, 16, ST, IOB>(a, s);
    if (P == 64 && N == 64) return launch_w<64, 64, ST, IOB>(a, s);
    if (P == 64 && N == 128) return launch_w<64, 128, ST, IOB>(a, s);
    if (P == 128 && N == 128) return launch_w<128, 128, ST, IOB>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace replay
