// verify_wide.hip -- speculative verify of windows of up to 16 drafts on the
// matrix cores, reading the float32 checkpoint or a bf16, e4m3 or MX FP4
// copy; bf16 io (replay_verify takes it from W = kWideFrom on) or float32 io
// (queries kept in float32, every product on v_mfma_f32_16x16x4_f32;
// replay_verify takes it past the register kernel's 8).
//
// The same outputs as the verify kernel of decode_impl.h: for the W newest
// ring entries t_w = count-W+w of every (sequence, head)
//     y_w = abar_{t_w} (S q_{t_w}) + sum_{j<=t_w} s_{j,t_w} v_j (k_j . q_{t_w})
// against one read of the checkpoint (page "ReplaySSM: Cachear Inputs, No
// Estado", section "Paralelismo": every window position reads the same
// checkpoint and buffer, entry j visible to position t when j <= t; eq. "Ruta
// solo salida").  With W queries every state element enters W products; the
// register kernel's per-row partial sums grow with W (past eight they no
// longer fit), and here S Q^T is formed as a matrix product instead
// (wide_mx.h: coalesced tile reads, a per-wavefront transpose into the
// operand layout, MFMA against the window's queries in LDS), and the ring
// wavefront(s) form the ring term for the window (ring_mx.h).  Output D[p][w]
// sits in lane (4-row group, column w), register r -> row 16i + 4g + r, so
// each lane writes four consecutive outputs of one query.
#include "decode_impl.h"
#include "wide_mx.h"

namespace replay {

template <int P, int N, int ST, int LM, bool IOB>
struct WideShape : WideTile<P, N, ST> {
    static constexpr int NR = LM / 16;
    static constexpr int NT = WideTile<P, N, ST>::NTS + 64 * NR;
    static constexpr int TSF = N + 4;   // LDS row stride of float32 queries (float32 io), in floats
};

// The ring part for a window of W <= 16 positions, operands from the ring
// (as ring_wave_mx of the decode kernel, with the window size at run time;
// float32 io: the same layout with float operands).
template <int P, int N, int LM, bool IOB>
__device__ __forceinline__ void wide_ring_wave(const RingView &r, int lane, int j0, int b, int g, size_t bh,
                                               int base, int count, int W, float (*s_r)[P], float *s_abar) {
    using MX = MxRing<P, N, kWide, LM, IOB>;
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
        m.aj = r.a[dta_index(b, bh, r.H, L, sl)];
        m.dtj = r.dt[dta_index(b, bh, r.H, L, sl)];
    }
    if constexpr (IOB) {
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
    } else {
#pragma unroll
        for (int kb = 0; kb < MX::KB; ++kb) {
            const int c = MX::col(kb, lane);
            const int j = j0 + lr;
            const float *kr = static_cast<const float *>(r.k) + (gring + slot(j < count ? j : last)) * N + c;
            const float *qr = static_cast<const float *>(r.q) + (gring + slot(t0 + (lr < W ? lr : W - 1))) * N + c;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                m.kf[kb][hf] = *reinterpret_cast<const f32x4 *>(kr + 4 * hf);
                m.qf[kb][hf] = *reinterpret_cast<const f32x4 *>(qr + 4 * hf);
            }
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int j = j0 + 4 * lq + kk;
            const float *vr = static_cast<const float *>(r.v) + (hring + slot(j < count ? j : last)) * P;
#pragma unroll
            for (int pw = 0; pw < MX::PW; ++pw)
                m.vf[kk][pw] = *reinterpret_cast<const u32x2 *>(vr + 2 * MX::vword(pw, lane));
        }
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

template <int P, int N, int ST, int LM, bool IOB>
__global__ __launch_bounds__((WideShape<P, N, ST, LM, IOB>::NT)) void verify_wide_kernel(DecodeArgs args) {
    using WS = WideShape<P, N, ST, LM, IOB>;
    constexpr int NTS = WS::NTS, TS = WS::TS, NR = WS::NR, TSF = WS::TSF;
    using TE = typename WS::TE;

    // the window's queries, Q[w][n]: bf16 (bf16 io) or float32
    __shared__ __align__(16) TE s_Q[IOB ? kWide : 1][IOB ? TS : 8];
    __shared__ __align__(16) float s_Qf[IOB ? 1 : kWide][IOB ? 4 : TSF];
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
    WideRows<P, N, ST> rows;
    if (wave < NTS / 64) rows.load(args.S, bh * (size_t)(P * N), p0, lane, args.scale);
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
        wide_ring_wave<P, N, LM, IOB>(r, lane, 16 * blk, b, g, bh, base, count, W, s_r[blk], s_abar);
        __syncthreads();
        return;
    }
    {
        // the queries: row w of Q is ring entry count-W+w, zero for w >= W;
        // 16 bytes (8 bf16 or 4 floats) a thread, every load issued before any is used
        const size_t gring = ((size_t)b * r.G + g) * L;
        const int bmod = base % L;
        constexpr int QE = IOB ? 8 : 4;   // elements per 16 bytes
        constexpr int QP = kWide * N / QE, QI = (QP + NTS - 1) / NTS;
        uint4 qraw[QI];
#pragma unroll
        for (int i = 0; i < QI; ++i) {
            const int e = (i * NTS + tid < QP ? i * NTS + tid : QP - 1) * QE;
            const int w = e / N, n = e % N;
            const size_t qe = (gring + ring_slot(bmod, count - W + (w < W ? w : W - 1), L)) * N + n;
            if constexpr (IOB)
                qraw[i] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(r.q) + qe);
            else
                qraw[i] = *reinterpret_cast<const uint4 *>(static_cast<const float *>(r.q) + qe);
        }
#pragma unroll
        for (int i = 0; i < QI; ++i) {
            if (i * NTS + tid < QP) {
                const int e = (i * NTS + tid) * QE;
                const int w = e / N, n = e % N;
                const uint4 u = w < W ? qraw[i] : uint4{0u, 0u, 0u, 0u};
                if constexpr (IOB)
                    wide_put_q<P, N, ST>(s_Q, w, n, u);
                else
                    *reinterpret_cast<uint4 *>(&s_Qf[w][n]) = u;
            }
        }
    }
    __syncthreads();

    rows.transpose(s_T[WS::COAL ? wave : 0], lane);
    f32x4 acc;
    const uint8_t *rsc = static_cast<const uint8_t *>(args.scale) + (bh * P + p0 + 4 * lg) * WS::NB;   // FP4 rows
    if constexpr (!IOB)
        acc = rows.dot_f32q(s_Qf, lane, rsc);
    else if constexpr (ST == ST_FP4 && WS::BF)
        acc = rows.dot_mx(s_Q, lane, rsc);
    else
        acc = rows.dot(s_Q, lane);
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
            o[rr] = wide_out(ab, sc, acc[rr], rt);
        }
        *reinterpret_cast<f32x4 *>(&args.y[(((size_t)b * W + w) * H + h) * P + p0 + 4 * lg]) = o;
    }
}

template <int P, int N, int ST, bool IOB>
static hipError_t launch_wide_io(const DecodeArgs &a, hipStream_t s) {
    const unsigned blocks = (unsigned)((size_t)a.r.B * a.r.H);
    if (a.r.L <= 16)
        verify_wide_kernel<P, N, ST, 16, IOB><<<blocks, WideShape<P, N, ST, 16, IOB>::NT, 0, s>>>(a);
    else
        verify_wide_kernel<P, N, ST, kMaxRing, IOB><<<blocks, WideShape<P, N, ST, kMaxRing, IOB>::NT, 0, s>>>(a);
    return hipGetLastError();
}

template <int P, int N, int ST>
static hipError_t launch_wide_st(const DecodeArgs &a, hipStream_t s) {
    return a.r.io_bf16 ? launch_wide_io<P, N, ST, true>(a, s) : launch_wide_io<P, N, ST, false>(a, s);
}

template <int P, int N>
static hipError_t launch_wide_pn(int st, const DecodeArgs &a, hipStream_t s) {
    switch (st) {
        case ST_F32: return launch_wide_st<P, N, ST_F32>(a, s);
        case ST_BF16: return launch_wide_st<P, N, ST_BF16>(a, s);
        case ST_FP8: return launch_wide_st<P, N, ST_FP8>(a, s);
        case ST_FP4: return launch_wide_st<P, N, ST_FP4>(a, s);
        default: return hipErrorInvalidValue;
    }
}

bool verify_wide_supported(int st, const DecodeArgs &a) {
    return (st == ST_F32 || st == ST_BF16 || st == ST_FP8 || st == ST_FP4) && a.W >= 1 && a.W <= kMaxWideWindow &&
           a.W <= a.r.L;
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
