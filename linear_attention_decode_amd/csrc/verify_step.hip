// verify_step.hip -- one fused speculative-verify round for a float32
// checkpoint with bf16 io.
//
// For every (sequence, head), in one launch:
//   1. where the ring holds count >= max(flush_at, 1) entries, fold them into
//      the checkpoint by the state-and-output route (page "ReplaySSM: Cachear
//      Inputs, No Estado", section "Los dos caminos", eq. "Ruta estado y
//      salida"):  S_new = abar_c S0 + sum_j s_{j,c} v_j k_j^T, written back
//      once, and base = pos;
//   2. append the W drafts at ring positions pos .. pos+W-1;
//   3. score the drafts t_w = count'-W+w by the output-only route (eq. "Ruta
//      solo salida"; section "Paralelismo": every draft reads the same
//      checkpoint and buffer, entry j is visible to draft t when j <= t):
//        y_w = abar_{t_w} (S q_w) + sum_{j<=t_w} s_{j,t_w} v_j (k_j . q_w),
//      with S the checkpoint just read or just folded.
// The results equal those of the flush, append and verify kernels run in
// turn, bit for bit; the checkpoint is read once per round and written only
// where it folds.
//
// Workgroup = the streaming wavefronts (the head's tile, S q_w for every
// draft: register sums over the fused step's 16-byte chunks for W < kWideFrom,
// the matrix-core products of wide_mx.h from kWideFrom on) + 2 ring
// wavefronts:
//   term wavefront   group dots and ring term of the window on the matrix
//                    cores (ring_mx.h); entries kept from before the round
//                    come from the ring, the drafts from the inputs;
//   fold wavefront   the fold's segment weights and its s_j v_j / k_j staging
//                    in LDS, and the drafts' per-head ring entries (v, dt, a).
// Draft w goes to ring slot (pos + w) mod L.  When the ring folds, those slots
// can hold entries the fold still reads.  The fold wavefront reads the per-head
// entries before it writes the drafts' ones.  The group-shared q/k rows, which
// every head's fold wavefront reads, are written by the group's last ring
// wavefront to arrive; each ring wavefront arrives only once its loads have
// returned.  The pointer moves when the sequence's last group arrives.
#include "step_common.h"
#include "wide_mx.h"
#include "decode_impl.h"

namespace replay {

constexpr int kVsRing = 16;   // ring entries covered by one term wavefront (L <= 16)

// Term wavefront.  Entry j < keep is ring entry j; entry keep + d is draft d
// (keep = 0 when the ring folds).  Entries past the window are clamped to the
// newest draft, as the verify kernel clamps them to the newest ring entry, so
// the matrix-core sums equal that kernel's bit for bit.
template <int P, int N, int W>
__device__ __forceinline__ int vs_term_wave(const StepArgs &A, int lane, int b, int g, int h, size_t bh,
                                            int base, int keep, float (*s_r)[P], float *s_abar,
                                            float (*s_sw)[kVsRing]) {
    using MX = MxRing<P, N, W, kVsRing>;
    constexpr uint32_t ES = 2;
    const int L = A.L, H = A.H, G = A.G, count = keep + W;
    const size_t gring = ((size_t)b * G + g) * L;
    const size_t hring = bh * L;
    const int bmod = base % L;
    auto slot = [&](int j) { return ring_slot(bmod, j, L); };
    auto draft = [&](int j) {
        const int d = j - keep;
        return d < 0 ? 0 : (d < W ? d : W - 1);
    };
    const int lastr = keep > 0 ? keep - 1 : 0;   // clamp for ring loads (unused when keep == 0)
    const int lr = lane & 15, lq = lane >> 4;

    MX m;
    m.j0 = 0;
    {
        const bool old = lane < keep;
        const size_t i = old ? dta_index(b, bh, H, L, slot(lane)) : ((size_t)b * W + draft(lane)) * H + h;
        m.aj = (old ? A.ring_a : A.a)[i];
        m.dtj = (old ? A.ring_dt : A.dt)[i];
    }
#pragma unroll
    for (int kb = 0; kb < MX::KB; ++kb) {
        const int c = MX::col(kb, lane);
        const bool old = lr < keep;
        const uint16_t *krow = old ? static_cast<const uint16_t *>(A.ring_k) + (gring + slot(lr)) * N
                                   : static_cast<const uint16_t *>(A.k) + (((size_t)b * W + draft(lr)) * G + g) * N;
        m.ka[kb] = *reinterpret_cast<const uint4 *>(krow + c);
        const int w = lr < W ? lr : W - 1;
        m.qb[kb] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(A.q) +
                                                    (((size_t)b * W + w) * G + g) * N + c);
    }
    // v pairs: one load from the ring and one from the drafts, selected per entry
    const auto rres = make_rsrc(static_cast<const char *>(A.ring_v) + hring * P * ES, (uint32_t)(L * P * ES));
    const auto ires = make_rsrc(static_cast<const char *>(A.v) + ((size_t)b * W * H + h) * P * ES,
                                (uint32_t)(((W - 1) * H + 1) * P * ES));
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int j = 4 * lq + kk;
        const bool old = j < keep;
        const uint32_t rrow = (uint32_t)slot(old ? j : lastr) * P;
        const uint32_t irow = (uint32_t)(draft(j) * H) * P;
#pragma unroll
        for (int pw = 0; pw < MX::PW; ++pw) {
            const uint32_t e = 2 * MX::vword(pw, lane);
            const uint32_t wr = __builtin_amdgcn_raw_buffer_load_b32(rres, (rrow + e) * ES, 0, 0);
            const uint32_t wi = __builtin_amdgcn_raw_buffer_load_b32(ires, (irow + e) * ES, 0, 0);
            m.vw[kk][pw] = old ? wr : wi;
        }
    }
    // Arrival.  This wavefront reads no ring slot a draft is written to
    // while it matters: entries < keep lie before the drafts' slots (keep + W
    // <= L), and with keep == 0 the clamped ring values are not used.
    int prev = -1;
    if (lane == 0) prev = atomicAdd(&A.sync[((size_t)b * (G + 1) + g) * kSyncStride], 1);
    // the workgroup's first barrier, with this wavefront's loads in flight
    // (the scheduling barrier keeps the work on the loaded values below it,
    // so the wavefront does not wait for them before the barrier)
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (lane >= count) {
        m.aj = 1.f;
        m.dtj = 0.f;
    }
    const f32x4 dk = m.dots(lane);
    m.weights(lane, count, s_abar, s_sw);
    m.term(lane, dk, s_r, s_sw);
    return prev;
}

// Fold wavefront: the drafts' per-head ring entries, and (when folding) the
// c = cold entries' segment weights, s_fabar = abar_c, U[p][j] = s_{j,c} v_j[p]
// and K[j][n] = k_j[n], in the flush kernel's order of operations.
template <int P, int N, int W>
__device__ __forceinline__ int vs_fold_wave(const StepArgs &A, int lane, int b, int g, int h, size_t bh, int base,
                                            int pos, int cold, bool fold, float *s_fabar,
                                            float (*s_U)[kVsRing + 1], float (*s_K)[N]) {
    constexpr int LM = kVsRing;
    constexpr int TS = N / 8;
    constexpr int RPW = 64 / TS;
    constexpr int KI = (LM + RPW - 1) / RPW;
    constexpr int VR = (P + 63) / 64;
    constexpr int VWORDS = W * P / 2, VWPL = (VWORDS + 63) / 64;
    constexpr uint32_t ES = 2;
    const int L = A.L, H = A.H, G = A.G;
    const size_t gring = ((size_t)b * G + g) * L;
    const size_t hring = bh * L;
    const int bmod = base % L, pmod = pos % L;
    auto slot = [&](int j) { return ring_slot(bmod, j, L); };
    const int c = fold ? cold : 0;
    const int lastr = c > 0 ? c - 1 : 0;
    const int tl = lane % TS, te = lane / TS;

    // the drafts' v rows (as words) and dt, a
    uint32_t vd[VWPL];
#pragma unroll
    for (int i = 0; i < VWPL; ++i) {
        const int idx = lane + 64 * i < VWORDS ? lane + 64 * i : VWORDS - 1;
        const int w = idx / (P / 2), wd = idx % (P / 2);
        vd[i] = static_cast<const uint32_t *>(A.v)[(((size_t)b * W + w) * H + h) * (P / 2) + wd];
    }
    const int wl = lane < W ? lane : W - 1;
    const float a_d = A.a[((size_t)b * W + wl) * H + h], dt_d = A.dt[((size_t)b * W + wl) * H + h];

    // the folded entries (clamped to valid ones; values past c are not used)
    float aj = 1.f, dtj = 0.f;
    IoVec<true, 8> kraw[KI];
    IoVec<true, 1> vraw[VR][LM];
    if (fold) {
        const int sl = slot(lane < c ? lane : lastr);
        aj = A.ring_a[dta_index(b, bh, H, L, sl)];
        dtj = A.ring_dt[dta_index(b, bh, H, L, sl)];
#pragma unroll
        for (int i = 0; i < KI; ++i) {
            const int j = i * RPW + te;
            kraw[i].load(A.ring_k, (gring + slot(j < c ? j : lastr)) * N + tl * 8);
        }
        const auto vres = make_rsrc(static_cast<const char *>(A.ring_v) + hring * P * ES, (uint32_t)(L * P * ES));
#pragma unroll
        for (int rr = 0; rr < VR; ++rr) {
            const uint32_t voff = ((lane + 64 * rr) < P ? lane + 64 * rr : P - 1) * ES;
#pragma unroll
            for (int j = 0; j < LM; ++j)
                vraw[rr][j].load_buf(vres, voff, (uint32_t)slot(j < c ? j : lastr) * P * ES);
        }
    }
    // the workgroup's first barrier, with this wavefront's loads in flight
    // (the scheduling barrier keeps the work on the loaded values below it,
    // so the wavefront does not wait for them before the barrier)
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // Every load above has returned before this wavefront arrives or writes:
    // the drafts' slots can hold folded entries, and the group's last arrival
    // overwrites the q/k rows read here.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    int prev = -1;
    if (lane == 0) prev = atomicAdd(&A.sync[((size_t)b * (G + 1) + g) * kSyncStride], 1);

    // the drafts' per-head entries into slots (pos + w) mod L
#pragma unroll
    for (int i = 0; i < VWPL; ++i) {
        const int idx = lane + 64 * i;
        if (idx < VWORDS) {
            const int w = idx / (P / 2), wd = idx % (P / 2);
            static_cast<uint32_t *>(A.ring_v)[(hring + ring_slot(pmod, w, L)) * (P / 2) + wd] = vd[i];
        }
    }
    if (lane < W) {
        A.ring_dt[dta_index(b, bh, H, L, ring_slot(pmod, lane, L))] = dt_d;
        A.ring_a[dta_index(b, bh, H, L, ring_slot(pmod, lane, L))] = a_d;
    }

    if (fold) {
        float prod = dtj, run = 1.f, sw = 0.f, ab = 0.f;
#pragma unroll
        for (int m = 0; m < LM; ++m) {
            if (m < c) {
                const float am = bcast(aj, m);
                if (m > lane) prod *= am;
                run *= am;
                if (m == c - 1) {
                    sw = prod;
                    ab = run;
                }
            }
        }
        if (lane == 0) *s_fabar = ab;
#pragma unroll
        for (int j = 0; j < LM; ++j) {
            if (j < c) {
                const float sj = bcast(sw, j);
#pragma unroll
                for (int rr = 0; rr < VR; ++rr)
                    if (lane + 64 * rr < P) s_U[lane + 64 * rr][j] = sj * vraw[rr][j].value();
            }
        }
#pragma unroll
        for (int i = 0; i < KI; ++i) {
            const int j = i * RPW + te;
            if (j < c) {
                float kk[8];
                kraw[i].widen(kk);
#pragma unroll
                for (int e = 0; e < 8; ++e) s_K[j][tl * 8 + e] = kk[e];
            }
        }
    }
    return prev;
}

// The streaming wavefronts with the window's products on the matrix cores
// (W >= kWideFrom; wide_mx.h, the same code and operands as the matrix-core
// verify kernel, so a round equals the flush, append and verify calls bit
// for bit).  Wavefront i owns rows 16i..16i+15 of the head's tile.  The fold
// runs on whichever layout holds the rows, element by element in the flush
// kernel's order (abar_c S0, then the entries' products one after another),
// writes S_new there and takes the products from it.
template <int P, int N, int W, class QRows, class TRows>
__device__ __forceinline__ void verify_step_streamer_mx(const StepArgs &args, int tid, int lane, int wave, int b,
                                                        int g, int h, size_t bh, size_t tile, QRows s_Q, TRows T,
                                                        float (*s_r)[P], float *s_abar, float (*s_U)[kVsRing + 1],
                                                        float (*s_K)[N], float &s_fabar, int &s_route,
                                                        int &s_fcount) {
    using WT = WideTile<P, N, ST_F32>;
    constexpr int NTS = WT::NTS;
    const int H = args.H, G = args.G;
    const int p0 = 16 * wave;
    // the drafts' queries first (rows w < W of Q, 8 elements a thread; rows
    // past W zero): loads complete in order, so waiting for them before the
    // LDS write does not wait for the tile
    constexpr int QP = kWide * N / 8, QI = (QP + NTS - 1) / NTS;
    uint4 qraw[QI];
#pragma unroll
    for (int i = 0; i < QI; ++i) {
        const int e = (i * NTS + tid < QP ? i * NTS + tid : QP - 1) * 8;
        const int w = e / N, n = e % N;
        qraw[i] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(args.q) +
                                                  (((size_t)b * W + (w < W ? w : W - 1)) * G + g) * N + n);
    }
    asm volatile("" ::: "memory");
    WideRows<P, N, ST_F32> rows;
    rows.load(args.S, tile, p0, lane);
#pragma unroll
    for (int i = 0; i < QI; ++i) {
        if (i * NTS + tid < QP) {
            const int e = (i * NTS + tid) * 8;
            const int w = e / N, n = e % N;
            wide_put_q<P, N, ST_F32>(s_Q, w, n, w < W ? qraw[i] : uint4{0u, 0u, 0u, 0u});
        }
    }
    lds_barrier();   // the route, the queries
    const int route = s_route;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (route == 0) {
        rows.transpose(T, lane);
        acc = rows.dot(s_Q, lane);
    }
    lds_barrier();   // the ring terms and the fold's staging
    if (route == 2) {
        for (int i = tid; i < W * P; i += NTS)
            args.y[(((size_t)b * W + i / P) * H + h) * P + i % P] = __builtin_nanf("");
        return;
    }
    if (route == 1) {
        // fold: S_new = abar_c S0 + sum_j U[row][j] K[j][col], written once
        const float abar = s_fabar;
        const int c = s_fcount;
        rows.each_f32(lane, [&](f32x4 &x, int, int) {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] *= abar;
        });
#pragma unroll 1   // keeps the LDS operands of one entry in registers at a time
        for (int j = 0; j < c; ++j) {
            rows.each_f32(lane, [&](f32x4 &x, int r, int c0) {
                const f32x4 kk = *reinterpret_cast<const f32x4 *>(&s_K[j][c0]);
                const float u = s_U[p0 + r][j];
                x[0] = fmaf(u, kk.x, x[0]);
                x[1] = fmaf(u, kk.y, x[1]);
                x[2] = fmaf(u, kk.z, x[2]);
                x[3] = fmaf(u, kk.w, x[3]);
            });
        }
        rows.each_f32(lane, [&](f32x4 &x, int r, int c0) {
            __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(args.S + tile + (size_t)(p0 + r) * N + c0));
        });
        rows.transpose(T, lane);
        acc = rows.dot(s_Q, lane);
    }
    // D[p0 + 4 lg + rr][w = lane % 16]
    const int w = lane & 15, lg = lane >> 4;
    if (w < W) {
        const float ab = s_abar[w];
        f32x4 o;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) o[rr] = wide_out(ab, 1.0f, acc[rr], s_r[w][p0 + 4 * lg + rr]);
        *reinterpret_cast<f32x4 *>(&args.y[(((size_t)b * W + w) * H + h) * P + p0 + 4 * lg]) = o;
    }
}

// Waves per SIMD to ask the register allocator for: 8 (64 registers) for the
// 64 x 128 tile, which then fits: 61-63 registers for W = 2..5 (row pieces),
// a few spilled words for W = 1 and the matrix-core windows (measured faster
// than 67 registers at 7 waves); the other tiles fit or spill too much.
template <int P, int N>
constexpr int vs_waves() { return P == 64 && N == 128 ? 8 : 1; }

template <int P, int N, int W>
__global__ __launch_bounds__((StepShape<P, N>::NTS + 128)) __attribute__((amdgpu_waves_per_eu(vs_waves<P, N>()))) void verify_step_kernel(StepArgs args) {
    // the register route tiles the checkpoint as the register verify kernel
    // does for this window (decode_impl.h), so that their row sums agree
    using Sh = DecodeShape<P, N, ST_F32, W>;
    static_assert(Sh::NTS == StepShape<P, N>::NTS && Sh::VEC == 4, "verify tiling");
    constexpr int VEC = Sh::VEC, NTS = Sh::NTS, ITER = Sh::ITER, LPR = Sh::LPR, RPI = Sh::RPI;
    constexpr int PPL = Sh::PPL, RPL = Sh::RPL;
    constexpr int LM = kVsRing;
    using RR = RowReduce<RPL, LPR>;

    __shared__ float s_r[W][P];
    __shared__ float s_abar[W];
    __shared__ __align__(16) float s_sw[W][LM];
    __shared__ float s_U[P][LM + 1];
    __shared__ __align__(16) float s_K[LM][N];
    // the drafts' queries, widened: rows for the register sums (W < kWideFrom),
    // or the matrix cores' Q (16 rows, past W zero) and per-wavefront staging
    constexpr bool MX = W >= kWideFrom;
    using WT = WideTile<P, N, ST_F32>;
    __shared__ __align__(16) float s_q[MX ? 1 : W][N];
    __shared__ __align__(16) uint16_t s_Q[MX ? kWide : 1][WT::TS];
    __shared__ __align__(16) uint32_t s_T[MX && WT::COAL ? NTS / 64 : 1][16][WT::TROW];
    __shared__ float s_fabar;
    __shared__ int s_route;   // 0 keep the ring, 1 fold first, 2 error (sequence left unchanged)
    __shared__ int s_fcount;

    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int H = args.H, G = args.G, L = args.L;
    // (wave-uniform: the buffer descriptors built from them stay scalar)
    const int b = __builtin_amdgcn_readfirstlane(lid / H), h = __builtin_amdgcn_readfirstlane(lid % H);
    const int g = (h * G) / H;
    const int tid = threadIdx.x, lane = tid & 63;
    // wave-uniform role (scalar branches; the ring wavefronts' pointer reads
    // go through the scalar cache)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool streamer = wave < NTS / 64;
    const int rw = wave - NTS / 64;
    const size_t bh = (size_t)b * H + h;
    const size_t tile = bh * (size_t)(P * N);
    const int jp = tid % LPR;   // piece of a row: chunk i covers columns VEC * (jp + LPR * (i % PPL))

    // Only the ring wavefronts read the pointer (each arrives after its
    // read).  They publish the route in LDS at a first barrier, which the
    // streaming wavefronts reach with their tile loads in flight; knowing the
    // route before the sums lets the route without a fold release each tile
    // chunk as it is used.  The two roles run in disjoint branches (each
    // with both barriers), so neither role's registers are live in the
    // other's code.
    if (streamer) {
      if constexpr (MX) {
        verify_step_streamer_mx<P, N, W>(args, tid, lane, wave, b, g, h, bh, tile, s_Q, s_T[WT::COAL ? wave : 0],
                                         s_r, s_abar, s_U, s_K, s_fabar, s_route, s_fcount);
      } else {
        using Fin = float[RR::FINAL][W];
        // The drafts' queries, widened into LDS (published by the first
        // barrier).  They are loaded before the tile: loads complete in
        // order, so the wait for them before the LDS write does not wait for
        // the tile, and the first barrier is not held up by it.
        constexpr int QP = W * N / 4;   // 4-element pieces
        constexpr int QI = (QP + NTS - 1) / NTS;
        IoVec<true, 4> qraw[QI];
#pragma unroll
        for (int i = 0; i < QI; ++i) {
            const int piece = tid + i * NTS < QP ? tid + i * NTS : QP - 1;
            const int w = piece / (N / 4), c = (piece % (N / 4)) * 4;
            qraw[i].load(args.q, (((size_t)b * W + w) * G + g) * N + c);
        }
        // (the empty asm keeps the compiler from moving the query loads
        // past the tile loads; lanes past the last piece repeat it, so the
        // loads and LDS writes are unconditional and stay in place)
        asm volatile("" ::: "memory");
        Chunk<ST_F32, VEC> ch[ITER];
#pragma unroll
        for (int i = 0; i < ITER; ++i) ch[i].load(args.S, tile + (size_t)Sh::offset(i, tid));
#pragma unroll
        for (int i = 0; i < QI; ++i) {
            const int piece = tid + i * NTS < QP ? tid + i * NTS : QP - 1;
            const int w = piece / (N / 4), c = (piece % (N / 4)) * 4;
            float qf[4];
            qraw[i].widen(qf);
            *reinterpret_cast<f32x4 *>(&s_q[w][c]) = f32x4{qf[0], qf[1], qf[2], qf[3]};
        }
        // S q_w for every draft, one draft at a time (each draft's partial
        // sums reduced before the next draft's are formed)
        auto sums = [&](const auto &tile_chunk, Fin &fin) {
#pragma unroll
            for (int w = 0; w < W; ++w) {
                f32x4 qp[PPL];
#pragma unroll
                for (int u = 0; u < PPL; ++u) qp[u] = *reinterpret_cast<const f32x4 *>(&s_q[w][VEC * (jp + LPR * u)]);
                float part[RPL][1];
#pragma unroll
                for (int rr = 0; rr < RPL; ++rr) {
                    f32x4 xp[PPL];
#pragma unroll
                    for (int u = 0; u < PPL; ++u) {
                        float x[VEC];
                        tile_chunk(rr * PPL + u, x);
                        xp[u] = f32x4{x[0], x[1], x[2], x[3]};
                    }
                    part[rr][0] = pieces_dot<PPL>(xp, qp);
                }
                RR::template run<1>(part, lane);
#pragma unroll
                for (int e = 0; e < RR::FINAL; ++e) fin[e][w] = part[e][0];
            }
        };
        Fin fin;
        lds_barrier();
        const int route = s_route;
        if (route == 0) sums([&](int i, float *x) { ch[i].widen(x, 1.0f); }, fin);
        lds_barrier();
        if (route == 2) {
            for (int i = tid; i < W * P; i += NTS)
                args.y[(((size_t)b * W + i / P) * H + h) * P + i % P] = __builtin_nanf("");
            return;
        }
        if (route == 1) {
            // fold: S_new = abar_c S0 + sum_j U[row][j] K[j][col], written once
            const float abar = s_fabar;
            float x[ITER][VEC];
#pragma unroll
            for (int i = 0; i < ITER; ++i) {
                ch[i].widen(x[i], 1.0f);
#pragma unroll
                for (int e = 0; e < VEC; ++e) x[i][e] *= abar;
            }
            const int c = s_fcount;
#pragma unroll 1   // keeps the LDS operands of one entry in registers at a time
            for (int j = 0; j < c; ++j) {
                float uu[RPL];
#pragma unroll
                for (int rr = 0; rr < RPL; ++rr) uu[rr] = s_U[rr * RPI + tid / LPR][j];
#pragma unroll
                for (int q = 0; q < PPL; ++q) {
                    const f32x4 kk = *reinterpret_cast<const f32x4 *>(&s_K[j][VEC * (jp + LPR * q)]);
#pragma unroll
                    for (int rr = 0; rr < RPL; ++rr) {
                        const int i = rr * PPL + q;
                        x[i][0] = fmaf(uu[rr], kk.x, x[i][0]);
                        x[i][1] = fmaf(uu[rr], kk.y, x[i][1]);
                        x[i][2] = fmaf(uu[rr], kk.z, x[i][2]);
                        x[i][3] = fmaf(uu[rr], kk.w, x[i][3]);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < ITER; ++i) {
                f32x4 o = {x[i][0], x[i][1], x[i][2], x[i][3]};
                // (plain stores: with 8-row store instructions they measured
                // faster than non-temporal ones, 133-135 against 137 us a round)
                *reinterpret_cast<f32x4 *>(args.S + tile + (size_t)Sh::offset(i, tid)) = o;
            }
            sums([&](int i, float *xo) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) xo[e] = x[i][e];
            }, fin);
        }
        if (RR::writer(lane)) {
            const int hi = RR::halving_index(lane);
#pragma unroll
            for (int e = 0; e < RR::FINAL; ++e) {
                const int row = (e + RR::FINAL * hi) * RPI + tid / LPR;
#pragma unroll
                for (int w = 0; w < W; ++w)
                    args.y[(((size_t)b * W + w) * H + h) * P + row] = s_abar[w] * fin[e][w] + s_r[w][row];
            }
        }
      }
    } else {
        const int base = args.base[b];
        int pos = args.pos[b];
        if (args.n_reject) {
            // the previous round's rollback first, as replay_rollback applies
            // it (page "ReplaySSM: Cachear Inputs, No Estado", "Rollback":
            // the pointer moves back); out of range: flagged, pointer kept
            const int r = args.n_reject[b];
            if (r < 0 || r > pos - base) {
                if (rw == 0 && lane == 0) raise_seq_error(args.err, b, REPLAY_SEQERR_ROLLBACK_RANGE);
            } else {
                pos -= r;
            }
        }
        const int cold = pos - base;
        const int need = args.flush_at > 1 ? args.flush_at : 1;
        const bool fold = cold >= need;
        const int keep = fold ? 0 : cold;
        const int err = keep + W > L ? REPLAY_SEQERR_RING_OVERFLOW
                                     : ((long long)pos + W > 2147483647LL ? REPLAY_SEQERR_POS_OVERFLOW : 0);
        if (rw == 0 && lane == 0) {
            s_route = err ? 2 : (fold ? 1 : 0);
            s_fcount = fold ? cold : 0;
            if (err) raise_seq_error(args.err, b, err);
        }
        // the first barrier: inside the ring functions, once their loads are issued
        int prev = -1;
        if (err) {
            lds_barrier();
        } else {
            if (rw == 0)
                prev = vs_term_wave<P, N, W>(args, lane, b, g, h, bh, base, keep, s_r, s_abar, s_sw);
            else
                prev = vs_fold_wave<P, N, W>(args, lane, b, g, h, bh, base, pos, cold, fold, &s_fabar, s_U, s_K);
        }
        // LDS-only barrier: the ring writes and arrival atomics finish in the background
        lds_barrier();
        if (__shfl(prev, 0) == 2 * (H / G) - 1) {
            // Last ring wavefront of the group to arrive: every ring wavefront
            // of the group has read what it reads from the ring, so the
            // drafts' q/k rows go into slots (pos + w) mod L now.  Then the
            // group arrives at the sequence's counter; the last group moves
            // the pointer.
            const size_t gring = ((size_t)b * G + g) * L;
            const int pmod = pos % L;
            constexpr int RW = RowWords<N, true>::WORDS;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                RowWords<N, true> qrow, krow;
                const size_t in = (((size_t)b * W + w) * G + g) * N * 2;
                qrow.load(static_cast<const char *>(args.q) + in, lane);
                krow.load(static_cast<const char *>(args.k) + in, lane);
                const size_t off = (gring + ring_slot(pmod, w, L)) * (size_t)RW * 4;
                qrow.store(static_cast<char *>(args.ring_q) + off, lane);
                krow.store(static_cast<char *>(args.ring_k) + off, lane);
            }
            if (lane == 0) {
                int32_t *seq = args.sync + (size_t)b * (G + 1) * kSyncStride;
                atomicExch(seq + (size_t)g * kSyncStride, 0);
                if (atomicAdd(seq + (size_t)G * kSyncStride, 1) == G - 1) {
                    atomicExch(seq + (size_t)G * kSyncStride, 0);
                    if (fold) args.base[b] = pos;
                    args.pos[b] = pos + W;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// The same round when the outputs read a low-precision copy (e4m3 or MX FP4)
// of the float32 master (separated precisions; page "ReplaySSM: Cache SSM
// Inputs, Not State", Abstract: output-only verification with a
// low-precision checkpoint serving the outputs, the higher-precision one
// taking the updates).  Equivalent to replay_flush(flush_at) (fold into the
// master, rewrite the copy), replay_append(W), replay_verify(W) from the
// copy, bit for bit:
//   - a round without a fold scores the drafts from the copy with the
//     register verify kernel's tiling and sums (decode_impl.h: bf16-pair
//     dot products of the codes, the e4m3 head scale or the FP4 block scales
//     applied as there);
//   - a folding head reads the master instead, folds it as the flush kernel
//     does (same tiling and order), writes the master and the new copy with
//     the flush kernel's quantisers (e4m3: one scale per head = amax / 448;
//     FP4: E8M0 scale per 32 values), stages the new codes in LDS and scores
//     the drafts from them with the same tiling and sums as the verify kernel
//     reading that copy.
// The ring wavefronts are the float32 round's (term, fold).  Four barriers:
// route; ring terms and fold staging; the e4m3 head maximum; the staged codes.
template <int P, int N, int ST>
struct VsCopyShape {
    using C = DecodeShape<P, N, ST, 2>;   // the verify kernel's copy tiling (any window past 1)
    using M = StepShape<P, N>;            // the fold's master tiling (the flush kernel's)
    static constexpr int NTS = M::NTS;
    static constexpr bool OK = (int)C::NTS == (int)M::NTS;
    static constexpr int CODE_BYTES = ST == ST_FP4 ? P * N / 2 : P * N;
};

template <int P, int N, int ST, int W>
__global__ __launch_bounds__((VsCopyShape<P, N, ST>::NTS + 128))
__attribute__((amdgpu_waves_per_eu(8))) void verify_step_copy_kernel(StepArgs args) {
    using VS = VsCopyShape<P, N, ST>;
    using SC = DecodeShape<P, N, ST, W>;
    using SM = typename VS::M;
    static_assert(VS::OK && (int)SC::NTS == VS::NTS, "copy and master tilings need the same streaming threads");
    constexpr int NTS = VS::NTS;
    constexpr int CVEC = SC::VEC, CITER = SC::ITER, CLPR = SC::LPR, CRPI = SC::RPI;
    constexpr int MVEC = SM::VEC, MITER = SM::ITER, MLPR = SM::LPR, MRPI = SM::RPI;
    constexpr int LM = kVsRing;
    using RR = RowReduce<CITER, CLPR>;
    using Ch = Chunk<ST, CVEC>;

    __shared__ float s_r[W][P];
    __shared__ float s_abar[W];
    __shared__ __align__(16) float s_sw[W][LM];
    __shared__ float s_U[P][LM + 1];
    __shared__ __align__(16) float s_K[LM][N];
    __shared__ __align__(16) uint8_t s_code[VS::CODE_BYTES];          // a folded head's new codes
    __shared__ uint8_t s_scl[ST == ST_FP4 ? P * N / 32 : 4];          // and its FP4 block scales
    __shared__ float s_red[NTS / 64];
    __shared__ __align__(16) uint32_t s_qw[W * N / 2];                // the drafts' query rows, bf16 pairs
    __shared__ float s_fabar;
    __shared__ int s_route;   // 0 keep the ring, 1 fold first, 2 error (sequence left unchanged)
    __shared__ int s_fcount;

    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int H = args.H, G = args.G, L = args.L;
    const int b = __builtin_amdgcn_readfirstlane(lid / H), h = __builtin_amdgcn_readfirstlane(lid % H);
    const int g = (h * G) / H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool streamer = wave < NTS / 64;
    const int rw = wave - NTS / 64;
    const size_t bh = (size_t)b * H + h;
    const size_t tile = bh * (size_t)(P * N);

    if (streamer) {
        // the drafts' query rows (bf16 pairs) into LDS, published by the first
        // barrier; they are loaded before the copy tile (loads complete in
        // order, so the wait before the LDS write does not wait for the tile)
        constexpr int QW = CVEC / 2;
        constexpr int QROW = N / 2, QALL = W * QROW, QI = (QALL + NTS - 1) / NTS;
        const int ccol0 = (tid % CLPR) * CVEC;
        uint32_t qword[QI];
#pragma unroll
        for (int i = 0; i < QI; ++i) {
            const int k = tid + i * NTS < QALL ? tid + i * NTS : QALL - 1;
            qword[i] = reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(args.q) +
                                                          (((size_t)b * W + k / QROW) * G + g) * N)[k % QROW];
        }
        asm volatile("" ::: "memory");
        Ch cc[CITER];
#pragma unroll
        for (int i = 0; i < CITER; ++i) {
            if constexpr (ST == ST_FP4)
                cc[i].load_mx(args.copy, args.copy_scale, tile + (size_t)(i * NTS + tid) * CVEC);
            else
                cc[i].load(args.copy, tile + (size_t)(i * NTS + tid) * CVEC);
        }
#pragma unroll
        for (int i = 0; i < QI; ++i)
            if (tid + i * NTS < QALL) s_qw[tid + i * NTS] = qword[i];
        float part[CITER][W];
        // each partial sum as the verify kernel forms it (one draft's words at a time here)
        auto sums = [&]() {
#pragma unroll
            for (int w = 0; w < W; ++w) {
                uint32_t qw[QW];
#pragma unroll
                for (int e = 0; e < QW; ++e) qw[e] = s_qw[w * QROW + ccol0 / 2 + e];
#pragma unroll
                for (int i = 0; i < CITER; ++i) {
                    float acc = cc[i].dot_bf16(qw);
                    if constexpr (ST == ST_FP4) acc = ldexpf(acc, cc[i].se);   // the block's scale, exact
                    part[i][w] = acc;
                }
            }
            RR::template run<W>(part, lane);
        };
        // y_w = abar_w (scale * sums) + ring term, as the verify kernel writes it
        auto emit = [&](float sc) {
            if (RR::writer(lane)) {
                const int hi = RR::halving_index(lane);
#pragma unroll
                for (int e = 0; e < RR::FINAL; ++e) {
                    const int row = (e + RR::FINAL * hi) * CRPI + tid / CLPR;
#pragma unroll
                    for (int w = 0; w < W; ++w)
                        args.y[(((size_t)b * W + w) * H + h) * P + row] = s_abar[w] * (sc * part[e][w]) + s_r[w][row];
                }
            }
        };
        lds_barrier();   // 1: the route, the queries
        const int route = s_route;
        // a folding head reads the master as soon as the route is known (its
        // loads fly while the ring wavefronts stage the fold)
        f32x4 x[MITER];   // the master chunks, folded in place
        if (route == 0) {
            sums();
        } else if (route == 1) {
#pragma unroll
            for (int i = 0; i < MITER; ++i)
                x[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(args.S + tile + (size_t)(i * NTS + tid) * MVEC));
        }
        lds_barrier();   // 2: the ring terms and the fold's staging
        // a round without a fold is finished here (its sums need not live on)
        if (route == 0) emit(ST == ST_FP8 ? static_cast<const float *>(args.copy_scale)[bh] : 1.0f);
        float sc = 1.0f;   // e4m3: the new head scale
        const int mcol0 = (tid % MLPR) * MVEC;
        if (route == 1) {
            // fold the master as the flush kernel does: x = abar_c S0, then the
            // entries' products one after another
            const float abar = s_fabar;
#pragma unroll
            for (int i = 0; i < MITER; ++i)
#pragma unroll
                for (int e = 0; e < MVEC; ++e) x[i][e] *= abar;
            const int c = s_fcount;
#pragma unroll 1
            for (int j = 0; j < c; ++j) {
                const f32x4 kk = *reinterpret_cast<const f32x4 *>(&s_K[j][mcol0]);
#pragma unroll
                for (int i = 0; i < MITER; ++i) {
                    const float u = s_U[i * MRPI + tid / MLPR][j];
                    x[i][0] = fmaf(u, kk.x, x[i][0]);
                    x[i][1] = fmaf(u, kk.y, x[i][1]);
                    x[i][2] = fmaf(u, kk.z, x[i][2]);
                    x[i][3] = fmaf(u, kk.w, x[i][3]);
                }
            }
#pragma unroll
            for (int i = 0; i < MITER; ++i)
                __builtin_nontemporal_store(x[i], reinterpret_cast<f32x4 *>(args.S + tile + (size_t)(i * NTS + tid) * MVEC));
            if constexpr (ST == ST_FP8) {
                float amax = 0.f;
#pragma unroll
                for (int i = 0; i < MITER; ++i)
#pragma unroll
                    for (int e = 0; e < MVEC; ++e) amax = fmaxf(amax, fabsf(x[i][e]));
#pragma unroll
                for (int bit = 5; bit >= 0; --bit) amax = fmaxf(amax, lane_partner(amax, bit));
                if (lane == 0) s_red[wave] = amax;
            }
        }
        lds_barrier();   // 3: the head's maximum (e4m3)
        if (route == 1) {
            // the new copy, written to memory and staged in LDS
            if constexpr (ST == ST_FP8) {
                float amax = s_red[0];
#pragma unroll
                for (int i = 1; i < NTS / 64; ++i) amax = fmaxf(amax, s_red[i]);
                const float sig = amax > 0.f ? amax / 448.0f : 1.0f;   // correctly rounded divide
                const ScaleDiv dv(sig);
                uint8_t *cp = static_cast<uint8_t *>(const_cast<void *>(args.copy)) + tile;
                dv.run([&](auto div) {
#pragma unroll
                    for (int i = 0; i < MITER; ++i) {
                        const uint32_t o = f32x4_to_fp8(div(x[i][0]), div(x[i][1]), div(x[i][2]), div(x[i][3]));
                        const size_t e0 = (size_t)(i * NTS + tid) * MVEC;
                        __builtin_nontemporal_store(o, reinterpret_cast<uint32_t *>(cp + e0));
                        *reinterpret_cast<uint32_t *>(&s_code[e0]) = o;
                    }
                });
                if (tid == 0) static_cast<float *>(const_cast<void *>(args.copy_scale))[bh] = sig;
                sc = sig;
            } else {
                uint8_t *cp = static_cast<uint8_t *>(const_cast<void *>(args.copy));
                uint8_t *scl = static_cast<uint8_t *>(const_cast<void *>(args.copy_scale));
#pragma unroll
                for (int i = 0; i < MITER; ++i) {
                    float amax = fmaxf(fmaxf(fabsf(x[i][0]), fabsf(x[i][1])), fmaxf(fabsf(x[i][2]), fabsf(x[i][3])));
#pragma unroll
                    for (int bit = 2; bit >= 0; --bit) amax = fmaxf(amax, lane_partner(amax, bit));
                    const int se = mxfp4_block_exp(amax);
                    const size_t e0 = (size_t)(i * NTS + tid) * MVEC;   // within the head's tile
                    const uint16_t code = mxfp4_codes4(x[i][0], x[i][1], x[i][2], x[i][3], se);
                    *reinterpret_cast<uint16_t *>(cp + (tile + e0) / 2) = code;
                    *reinterpret_cast<uint16_t *>(&s_code[e0 / 2]) = code;
                    if ((tid & 7) == 0) {
                        scl[(tile + e0) / 32] = (uint8_t)(se + 127);
                        s_scl[e0 / 32] = (uint8_t)(se + 127);
                    }
                }
            }
        }
        lds_barrier();   // 4: the staged codes
        if (route == 2) {
            for (int i = tid; i < W * P; i += NTS)
                args.y[(((size_t)b * W + i / P) * H + h) * P + i % P] = __builtin_nanf("");
            return;
        }
        if (route == 1) {
            // the new codes in the copy tiling, as the verify kernel reads them
#pragma unroll
            for (int i = 0; i < CITER; ++i) {
                const size_t e = (size_t)(i * NTS + tid) * CVEC;   // within the head's tile
                if constexpr (ST == ST_FP4) {
                    static_assert(CVEC == 8 || CVEC == 4, "FP4 chunks of 4 or 2 bytes");
                    if constexpr (CVEC == 8)
                        cc[i].raw[0] = *reinterpret_cast<const uint32_t *>(&s_code[e / 2]);
                    else
                        cc[i].raw[0] = *reinterpret_cast<const uint16_t *>(&s_code[e / 2]);
                    cc[i].se = (int)s_scl[e / 32] - 127;
                } else {
#pragma unroll
                    for (int k = 0; k < CVEC / 4; ++k) cc[i].raw[k] = *reinterpret_cast<const uint32_t *>(&s_code[e + 4 * k]);
                }
            }
            sums();
            emit(sc);
        }
    } else {
        const int base = args.base[b];
        int pos = args.pos[b];
        if (args.n_reject) {
            // the previous round's rollback first, as replay_rollback applies
            // it (page "ReplaySSM: Cachear Inputs, No Estado", "Rollback":
            // the pointer moves back); out of range: flagged, pointer kept
            const int r = args.n_reject[b];
            if (r < 0 || r > pos - base) {
                if (rw == 0 && lane == 0) raise_seq_error(args.err, b, REPLAY_SEQERR_ROLLBACK_RANGE);
            } else {
                pos -= r;
            }
        }
        const int cold = pos - base;
        const int need = args.flush_at > 1 ? args.flush_at : 1;
        const bool fold = cold >= need;
        const int keep = fold ? 0 : cold;
        const int err = keep + W > L ? REPLAY_SEQERR_RING_OVERFLOW
                                     : ((long long)pos + W > 2147483647LL ? REPLAY_SEQERR_POS_OVERFLOW : 0);
        if (rw == 0 && lane == 0) {
            s_route = err ? 2 : (fold ? 1 : 0);
            s_fcount = fold ? cold : 0;
            if (err) raise_seq_error(args.err, b, err);
        }
        int prev = -1;
        if (err) {
            lds_barrier();   // 1
        } else {
            if (rw == 0)
                prev = vs_term_wave<P, N, W>(args, lane, b, g, h, bh, base, keep, s_r, s_abar, s_sw);
            else
                prev = vs_fold_wave<P, N, W>(args, lane, b, g, h, bh, base, pos, cold, fold, &s_fabar, s_U, s_K);
        }
        lds_barrier();   // 2
        lds_barrier();   // 3
        lds_barrier();   // 4
        if (__shfl(prev, 0) == 2 * (H / G) - 1) {
            // last ring wavefront of the group: the drafts' q/k rows, then the
            // group arrives at the sequence's counter (as in the float32 round)
            const size_t gring = ((size_t)b * G + g) * L;
            const int pmod = pos % L;
            constexpr int RW = RowWords<N, true>::WORDS;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                RowWords<N, true> qrow, krow;
                const size_t in = (((size_t)b * W + w) * G + g) * N * 2;
                qrow.load(static_cast<const char *>(args.q) + in, lane);
                krow.load(static_cast<const char *>(args.k) + in, lane);
                const size_t off = (gring + ring_slot(pmod, w, L)) * (size_t)RW * 4;
                qrow.store(static_cast<char *>(args.ring_q) + off, lane);
                krow.store(static_cast<char *>(args.ring_k) + off, lane);
            }
            if (lane == 0) {
                int32_t *seq = args.sync + (size_t)b * (G + 1) * kSyncStride;
                atomicExch(seq + (size_t)g * kSyncStride, 0);
                if (atomicAdd(seq + (size_t)G * kSyncStride, 1) == G - 1) {
                    atomicExch(seq + (size_t)G * kSyncStride, 0);
                    if (fold) args.base[b] = pos;
                    args.pos[b] = pos + W;
                }
            }
        }
    }
}

template <int P, int N, int ST, int W>
static hipError_t launch_vsc(const StepArgs &a, hipStream_t s) {
    if constexpr (VsCopyShape<P, N, ST>::OK) {
        const unsigned blocks = (unsigned)((size_t)a.B * a.H);
        verify_step_copy_kernel<P, N, ST, W><<<blocks, VsCopyShape<P, N, ST>::NTS + 128, 0, s>>>(a);
        return hipGetLastError();
    } else {
        return hipErrorInvalidValue;
    }
}

template <int P, int N, int ST>
static hipError_t launch_vsc_w(const StepArgs &a, hipStream_t s) {
    switch (a.W) {
        case 2: return launch_vsc<P, N, ST, 2>(a, s);
        case 3: return launch_vsc<P, N, ST, 3>(a, s);
        case 4: return launch_vsc<P, N, ST, 4>(a, s);
        case 5: return launch_vsc<P, N, ST, 5>(a, s);
        default: return hipErrorInvalidValue;
    }
}

bool verify_step_copy_fused(int P, int N, const StepArgs &a) {
    const bool shape = (P == 16 && N == 16) || (P == 64 && N == 64) || (P == 64 && N == 128);
    const bool copy = a.copy_st == ST_FP8 || a.copy_st == ST_FP4;
    // windows of 2 to 5 (a window of 1 is the several-head decode kernel's
    // tiling; from kWideFrom the e4m3 verify runs on the matrix cores)
    return shape && copy && a.S && a.io_bf16 && a.L <= kVsRing && a.W >= 2 && a.W < kWideFrom && a.W <= a.L;
}

hipError_t launch_verify_step_copy(int P, int N, const StepArgs &a, hipStream_t s) {
    if (!verify_step_copy_fused(P, N, a)) return hipErrorInvalidValue;
    const bool fp8 = a.copy_st == ST_FP8;
    if (P == 16 && N == 16) return fp8 ? launch_vsc_w<16, 16, ST_FP8>(a, s) : launch_vsc_w<16, 16, ST_FP4>(a, s);
    if (P == 64 && N == 64) return fp8 ? launch_vsc_w<64, 64, ST_FP8>(a, s) : launch_vsc_w<64, 64, ST_FP4>(a, s);
    return fp8 ? launch_vsc_w<64, 128, ST_FP8>(a, s) : launch_vsc_w<64, 128, ST_FP4>(a, s);
}

template <int P, int N, int W>
static hipError_t launch_vs(const StepArgs &a, hipStream_t s) {
    const unsigned blocks = (unsigned)((size_t)a.B * a.H);
    verify_step_kernel<P, N, W><<<blocks, StepShape<P, N>::NTS + 128, 0, s>>>(a);
    return hipGetLastError();
}

template <int P, int N>
static hipError_t launch_vs_w(const StepArgs &a, hipStream_t s) {
    switch (a.W) {
        case 1: return launch_vs<P, N, 1>(a, s);
        case 2: return launch_vs<P, N, 2>(a, s);
        case 3: return launch_vs<P, N, 3>(a, s);
        case 4: return launch_vs<P, N, 4>(a, s);
        case 5: return launch_vs<P, N, 5>(a, s);
        case 6: return launch_vs<P, N, 6>(a, s);
        case 7: return launch_vs<P, N, 7>(a, s);
        case 8: return launch_vs<P, N, 8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

bool verify_step_fused(int P, int N, const StepArgs &a) {
    const bool shape = (P == 16 && N == 16) || (P == 64 && N == 64) || (P == 64 && N == 128) || (P == 128 && N == 128);
    return shape && a.io_bf16 && a.L <= kVsRing && a.W >= 1 && a.W <= 8 && a.W <= a.L;
}

hipError_t launch_verify_step(int P, int N, const StepArgs &a, hipStream_t s) {
    if (!verify_step_fused(P, N, a)) return hipErrorInvalidValue;
    if (P == 16 && N == 16) return launch_vs_w<16, 16>(a, s);
    if (P == 64 && N == 64) return launch_vs_w<64, 64>(a, s);
    if (P == 64 && N == 128) return launch_vs_w<64, 128>(a, s);
    return launch_vs_w<128, 128>(a, s);
}

}  // namespace replay
