// step.hip -- one fused standard decode step for a float32 checkpoint.
//
// For every (sequence, head), in one launch: append this step's token to
// the ring, then either
//   output-only route  y = abar_t (S0 q) + sum_{j<=t} s_{j,t} v_j (k_j . q)
//   (page "ReplaySSM: Cachear Inputs, No Estado", section "Los dos caminos",
//   eq. "Ruta solo salida"), or, when the ring then holds count >= flush_at
//   entries, the state-and-output route that the flush needs (same section,
//   eq. "Ruta estado y salida"):
//     S_new = abar_c S0 + sum_j s_{j,c} v_j k_j^T   (written back once)
//     y     = S_new q
// with abar_t = prod_{m<=t} a_m, s_{j,t} = dt_j prod_{j<m<=t} a_m ("Decodificacion
// estandar": buffer the inputs, output by the output-only route, flush when
// the buffer is full).  The checkpoint is read once per step either way.
//
// Workgroup = 4 streaming wavefronts (8 for a 128 x 128 tile; the head's tile
// in 16-byte chunks) + 1 ring wavefront (decays, group dots, ring term or the
// rank-c staging).  The new token is taken from the inputs, so the streaming
// wavefronts never wait for the ring pointer.  One writer workgroup per
// sequence, after every compute workgroup in the grid, copies the token into
// the ring.  The pointer of a sequence moves when its last workgroup arrives
// (per-sequence counter).
#include "step_common.h"

namespace replay {

template <int P, int N, int LM, bool IOB>
__device__ __forceinline__ int step_ring_wave(const StepArgs &A, int lane, int b, int g, int h, size_t bh,
                                              int base, int cold, bool fold, float *s_r, float *s_abar,
                                              float (*s_U)[LM + 1], float (*s_K)[N]) {
    constexpr int TS = N / 8;
    constexpr int RPW = 64 / TS;
    constexpr int KI = (LM + RPW - 1) / RPW;
    constexpr int VR = (P + 63) / 64;
    const int L = A.L, count = cold + 1;
    const size_t gring = ((size_t)b * A.G + g) * L;
    const size_t hring = bh * L;
    const size_t gin = (size_t)b * A.G + g;
    const int bmod = base % L;
    auto slot = [&](int j) { return ring_slot(bmod, j, L); };
    const int lastr = cold > 0 ? cold - 1 : 0;   // clamp for ring loads (never used when cold == 0)
    const int tl = lane % TS, te = lane / TS;

    // 1. every load, issued before any value is used: this step's token
    // first, then the ring
    const float a_in = A.a[bh], dt_in = A.dt[bh];
    IoVec<IOB, 1> vnew[VR];
#pragma unroll
    for (int rr = 0; rr < VR; ++rr) vnew[rr].load(A.v, bh * P + ((lane + 64 * rr) < P ? lane + 64 * rr : P - 1));
    const int sla = slot(lane < cold ? lane : lastr);
    const float a_r = A.ring_a[dta_index(b, bh, A.H, L, sla)], dt_r = A.ring_dt[dta_index(b, bh, A.H, L, sla)];
    IoVec<IOB, 8> kraw[KI];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
        const int j = i * RPW + te;   // entries < cold from the ring, the rest from this step's k
        const bool old = j < cold;
        kraw[i].load(old ? A.ring_k : A.k, old ? (gring + slot(j)) * N + tl * 8 : gin * N + tl * 8);
    }
    IoVec<IOB, 8> qraw;
    qraw.load(A.q, gin * N + tl * 8);
    // ring values of entries < cold; the loads are unconditional from a
    // clamped, always-valid slot so that no branch or early wait sits between
    // them, and entry cold (this step's token) is selected at use
    constexpr uint32_t ES = IOB ? 2 : 4;
    const auto vres = make_rsrc(static_cast<const char *>(A.ring_v) + hring * P * ES, (uint32_t)(L * P * ES));
    IoVec<IOB, 1> vraw[VR][LM];
#pragma unroll
    for (int rr = 0; rr < VR; ++rr) {
        const uint32_t voff = ((lane + 64 * rr) < P ? lane + 64 * rr : P - 1) * ES;
#pragma unroll
        for (int j = 0; j < LM; ++j) vraw[rr][j].load_buf(vres, voff, (uint32_t)slot(j < cold ? j : lastr) * P * ES);
    }
    auto vval = [&](int rr, int j) { return j < cold ? vraw[rr][j].value() : vnew[rr].value(); };

    // Arrival of this workgroup (its pointer read is done: the loads above
    // depend on it).  Its result is needed only at the very end.
    int prev = -1;
    if (lane == 0) prev = atomicAdd(&A.sync[((size_t)b * (A.G + 1) + g) * kSyncStride], 1);

    // 3. decays of entries 0..count-1 (entry cold is this step's token)
    const float aj = lane < cold ? a_r : (lane == cold ? a_in : 1.f);
    const float dtj = lane < cold ? dt_r : (lane == cold ? dt_in : 0.f);
    float prod = dtj, run = 1.f, sw = 0.f, ab = 0.f;
#pragma unroll
    for (int m = 0; m < LM; ++m) {
        if (m < count) {
            const float am = bcast(aj, m);
            if (m > lane) prod *= am;
            run *= am;
            if (m == count - 1) {
                sw = prod;
                ab = run;
            }
        }
    }
    if (lane == 0) *s_abar = ab;

    if (!fold) {
        // output-only route: group dots, coefficients, ring term
        float cw = 0.f;
#pragma unroll
        for (int i = 0; i < KI; ++i) {
            float d = dot8(kraw[i], qraw);
            d = group_sum<TS>(d);
            const float moved = __shfl(d, (lane % RPW) * TS);
            if (lane / RPW == i) cw = moved;
        }
        const float coef = lane < count ? sw * cw : 0.f;
        float acc[VR];
#pragma unroll
        for (int rr = 0; rr < VR; ++rr) acc[rr] = 0.f;
#pragma unroll
        for (int j = 0; j < LM; ++j) {
            if (j < count) {
                const float cj = bcast(coef, j);
#pragma unroll
                for (int rr = 0; rr < VR; ++rr) acc[rr] = fmaf(cj, vval(rr, j), acc[rr]);
            }
        }
#pragma unroll
        for (int rr = 0; rr < VR; ++rr)
            if (lane + 64 * rr < P) s_r[lane + 64 * rr] = acc[rr];
    } else {
        // state-and-output route: stage U[p][j] = s_j v_j[p] and K[j][n] = k_j[n]
#pragma unroll
        for (int j = 0; j < LM; ++j) {
            if (j < count) {
                const float sj = bcast(sw, j);
#pragma unroll
                for (int rr = 0; rr < VR; ++rr)
                    if (lane + 64 * rr < P) s_U[lane + 64 * rr][j] = sj * vval(rr, j);
            }
        }
#pragma unroll
        for (int i = 0; i < KI; ++i) {
            const int j = i * RPW + te;
            if (j < count) {
                float kk[8];
                kraw[i].widen(kk);
#pragma unroll
                for (int e = 0; e < 8; ++e) s_K[j][tl * 8 + e] = kk[e];
            }
        }
    }

    return prev;
}

// Waves per SIMD to ask the register allocator for: 8 (the hardware maximum,
// 64 registers a lane) where the kernel fits without spilling to scratch
// (with bf16 io also for a 32-entry ring: 62 registers instead of 68 at 7
// waves), otherwise no request.
template <int P, int N, int LM, bool IOB>
constexpr int step_waves() {
    return (P * N <= 64 * 64 || (N == 128 && IOB)) && !(LM == 32 && P * N > 16 * 16 && !IOB) ? 8 : 1;
}

// Ring wavefronts of the fused step: two for a 32-entry ring with bf16 io
// (one per 16-entry block), else one.
template <int LM, bool IOB>
constexpr int step_ring_waves() { return IOB ? LM / 16 : 1; }

// Row splits of a head's tile: a 128-row tile with bf16 io is streamed by two
// workgroups of 64 rows each (4 + 1 wavefronts instead of 8 + 1, so six
// workgroups fit a CU where three did); each has its own ring wavefront(s)
// for its rows.
template <int P, bool IOB>
constexpr int step_row_splits() { return IOB && P == 128 ? 2 : 1; }

// One compute workgroup of the fused step: logical workgroup `bid` of the
// `ncomp` = B * H * RS of one layer.
// PH = rows of the head, RS = workgroups per head (rows P = PH / RS each).
template <int PH, int N, int LM, bool IOB, int RS>
__device__ __forceinline__ void step_body(const StepArgs &args, int bid, int ncomp) {
    constexpr int P = PH / RS;
    static_assert(RS == 1 || IOB, "row splits need the bf16 ring wavefront");
    using Sh = StepShape<P, N>;
    constexpr int VEC = Sh::VEC, NTS = Sh::NTS, ITER = Sh::ITER, LPR = Sh::LPR, RPI = Sh::RPI;
    constexpr int NR = step_ring_waves<LM, IOB>();
    using RR = RowReduce<ITER, LPR>;

    __shared__ float s_r[NR][P];
    __shared__ float s_abar;
    __shared__ int s_count;
    __shared__ float s_U[P][LM + 1];
    __shared__ __align__(16) float s_K[LM][N];
    __shared__ __align__(16) float s_sw[1][IOB ? LM : 4];

    const int H = args.H, L = args.L;
    const int lid = xcd_remap(bid, ncomp);
    const int b = lid / (H * RS), h = (lid / RS) % H, p0 = (lid % RS) * P;   // rows p0 .. p0+P-1
    const int g = (h * args.G) / H;
    const int tid = threadIdx.x, lane = tid & 63;
    // the role of this wavefront, as a wave-uniform value: the branches on it
    // are scalar, so the ring wavefronts' pointer reads go through the scalar
    // cache instead of queueing behind the tile loads of every wavefront on
    // the CU
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool streamer = wave < NTS / 64;
    const int rw = wave - NTS / 64;   // ring wavefront index
    const size_t bh = (size_t)b * H + h;
    const size_t tile = bh * (size_t)(PH * N) + (size_t)p0 * N;

    // Only the ring wavefronts read the pointer.  Each announces its arrival
    // once its ring loads are issued (the group's counter expects NR arrivals
    // per head), so the atomic's latency overlaps the rest of the work; the
    // streaming wavefronts learn the route (output-only, fold, or a
    // per-sequence error) from LDS after the barrier.  Each role loads only what it uses
    // inside its own branch, so the tile's registers are never live across
    // the ring wavefronts' code.
    __shared__ int s_route;   // 0 output-only, 1 fold, 2 error (sequence left unchanged)
    const int col0 = (tid % LPR) * VEC;
    Chunk<ST_F32, VEC> ch[ITER];
    IoVec<IOB, 4> qraw;
    float qv[VEC];
    float part[ITER][1];
    int pos = 0, prev = -1, route = 0;
    if (streamer) {
#pragma unroll
        for (int i = 0; i < ITER; ++i) ch[i].load(args.S, tile + (size_t)(i * NTS + tid) * VEC);
        qraw.load(args.q, ((size_t)b * args.G + g) * N + col0);
        qraw.widen(qv);
        // S0 q partials (used by the output-only route; cheap beside the loads)
#pragma unroll
        for (int i = 0; i < ITER; ++i) {
            float x[VEC];
            ch[i].widen(x, 1.0f);
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc = fmaf(x[e], qv[e], acc);
            part[i][0] = acc;
        }
        RR::template run<1>(part, lane);
    } else {
        const int base = args.base[b];
        pos = args.pos[b];
        const int cold = pos - base;
        const bool bad = cold + 1 > L || pos == 2147483647;
        const int need = args.flush_at > 1 ? args.flush_at : 1;
        route = bad ? 2 : (cold + 1 >= need ? 1 : 0);
        if (rw == 0 && lane == 0) {
            s_route = route;
            s_count = cold + 1;
            if (bad) raise_seq_error(args.err, b, cold + 1 > L ? REPLAY_SEQERR_RING_OVERFLOW : REPLAY_SEQERR_POS_OVERFLOW);
        }
        if (!bad) {
            if constexpr (IOB) {
                StepRingMx<P, N, LM, PH> sr;
                sr.load(args, lane, rw, b, g, h, bh, base, cold, p0);
                prev = sr.finish(args, lane, b, g, cold, route == 1, &s_r[rw], &s_abar, s_U, s_K,
                                 reinterpret_cast<float (*)[LM]>(&s_sw[0][0]));
            } else {
                prev = step_ring_wave<P, N, LM, IOB>(args, lane, b, g, h, bh, base, cold, route == 1, s_r[0],
                                                     &s_abar, s_U, s_K);
            }
        }
    }
    // LDS-only barrier: the ring wavefront's arrival atomic completes in the
    // background
    lds_barrier();
    if (streamer) route = s_route;

    if (streamer && route == 2) {
        for (int i = tid; i < P; i += NTS) args.y[bh * PH + p0 + i] = __builtin_nanf("");
    } else if (streamer) {
        if (route == 1) {
            const float abar = s_abar;
            float x[ITER][VEC];
#pragma unroll
            for (int i = 0; i < ITER; ++i) {
                ch[i].widen(x[i], 1.0f);
#pragma unroll
                for (int e = 0; e < VEC; ++e) x[i][e] *= abar;
            }
            const int count = s_count;
            for (int j = 0; j < count; ++j) {
                const f32x4 kk = *reinterpret_cast<const f32x4 *>(&s_K[j][col0]);
#pragma unroll
                for (int i = 0; i < ITER; ++i) {
                    const float u = s_U[i * RPI + tid / LPR][j];
                    x[i][0] = fmaf(u, kk.x, x[i][0]);
                    x[i][1] = fmaf(u, kk.y, x[i][1]);
                    x[i][2] = fmaf(u, kk.z, x[i][2]);
                    x[i][3] = fmaf(u, kk.w, x[i][3]);
                }
            }
#pragma unroll
            for (int i = 0; i < ITER; ++i) {
                f32x4 o = {x[i][0], x[i][1], x[i][2], x[i][3]};
                __builtin_nontemporal_store(o, reinterpret_cast<f32x4 *>(args.S + tile + (size_t)(i * NTS + tid) * VEC));
                float acc = 0.f;
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc = fmaf(x[i][e], qv[e], acc);
                part[i][0] = acc;
            }
            RR::template run<1>(part, lane);
        }
        if (RR::writer(lane)) {
            const int hi = RR::halving_index(lane);
            const float abar = s_abar;
#pragma unroll
            for (int e = 0; e < RR::FINAL; ++e) {
                const int row = (e + RR::FINAL * hi) * RPI + tid / LPR;
                float rt = s_r[0][row];
                if constexpr (NR == 2) rt += s_r[1][row];   // block 0 + block 1
                args.y[bh * PH + p0 + row] = route == 1 ? part[e][0] : abar * part[e][0] + rt;
            }
        }
    } else if (lane == 0 && prev == NR * RS * (H / args.G) - 1) {
        // Last ring wavefront of its group to arrive: the group arrives at
        // the sequence's counter (each ring wavefront arrived after its
        // pointer read).
        atomicExch(args.sync + ((size_t)b * (args.G + 1) + g) * kSyncStride, 0);
        step_seq_arrive(args, b, pos, route == 1);
    }
}

template <int PH, int N, int LM, bool IOB, int RS>
__global__ __launch_bounds__((StepShape<PH / RS, N>::NTS + 64 * step_ring_waves<LM, IOB>()))
__attribute__((amdgpu_waves_per_eu(step_waves<PH / RS, N, LM, IOB>()))) void step_kernel(StepArgs args) {
    const int ncomp = args.B * args.H * RS;   // compute workgroups; one writer per sequence follows
    if ((int)blockIdx.x >= ncomp) {
        step_token_writer<PH, N, IOB, true>(args, (int)blockIdx.x - ncomp, threadIdx.x, blockDim.x);
        return;
    }
    step_body<PH, N, LM, IOB, RS>(args, blockIdx.x, ncomp);
}

// The same step for n layers of one shape in one launch: the compute
// workgroups of layer 0, 1, ..., n-1, then the writer workgroups of every
// layer (B per layer).  The layers are independent; each keeps its own
// counters and pointers.
template <int PH, int N, int LM, bool IOB, int RS>
__global__ __launch_bounds__((StepShape<PH / RS, N>::NTS + 64 * step_ring_waves<LM, IOB>()))
__attribute__((amdgpu_waves_per_eu(step_waves<PH / RS, N, LM, IOB>()))) void step_layers_kernel(StepLayersArgs la) {
    const int B = la.l[0].B;
    const int ncomp = B * la.l[0].H * RS;
    const int bid = blockIdx.x, n = la.n;
    if (bid >= n * ncomp) {
        const int w = bid - n * ncomp;
        const int layer = w / B;
        step_token_writer<PH, N, IOB, true>(la.l[layer], w - layer * B, threadIdx.x, blockDim.x);
        return;
    }
    const int layer = bid / ncomp;
    step_body<PH, N, LM, IOB, RS>(la.l[layer], bid - layer * ncomp, ncomp);
}

template <int P, int N, int LM>
static hipError_t launch_layers_lm(const StepLayersArgs &a, hipStream_t s) {
    const StepArgs &a0 = a.l[0];
    if (a0.io_bf16) {
        constexpr int RS = step_row_splits<P, true>();
        const unsigned blocks = (unsigned)(((size_t)a0.B * a0.H * RS + a0.B) * a.n);
        step_layers_kernel<P, N, LM, true, RS>
            <<<blocks, StepShape<P / RS, N>::NTS + 64 * step_ring_waves<LM, true>(), 0, s>>>(a);
    } else {
        const unsigned blocks = (unsigned)(((size_t)a0.B * a0.H + a0.B) * a.n);
        step_layers_kernel<P, N, LM, false, 1>
            <<<blocks, StepShape<P, N>::NTS + 64 * step_ring_waves<LM, false>(), 0, s>>>(a);
    }
    return hipGetLastError();
}

int step_workgroups_per_layer(int P, const StepArgs &a) {
    return a.B * a.H * (a.io_bf16 ? (P == 128 ? step_row_splits<128, true>() : 1) : 1);
}

hipError_t launch_step_layers(int P, int N, const StepLayersArgs &a, hipStream_t s) {
    const bool small = a.l[0].L <= 16;
    if (P == 16 && N == 16) return small ? launch_layers_lm<16, 16, 16>(a, s) : launch_layers_lm<16, 16, kMaxRing>(a, s);
    if (P == 64 && N == 64) return small ? launch_layers_lm<64, 64, 16>(a, s) : launch_layers_lm<64, 64, kMaxRing>(a, s);
    if (P == 64 && N == 128) return small ? launch_layers_lm<64, 128, 16>(a, s) : launch_layers_lm<64, 128, kMaxRing>(a, s);
    if (P == 128 && N == 128)
        return small ? launch_layers_lm<128, 128, 16>(a, s) : launch_layers_lm<128, 128, kMaxRing>(a, s);
    return hipErrorInvalidValue;
}

template <int P, int N, int LM>
static hipError_t launch_lm(const StepArgs &a, hipStream_t s) {
    if (a.io_bf16) {
        constexpr int RS = step_row_splits<P, true>();
        const unsigned blocks = (unsigned)((size_t)a.B * a.H * RS + a.B);
        step_kernel<P, N, LM, true, RS>
            <<<blocks, StepShape<P / RS, N>::NTS + 64 * step_ring_waves<LM, true>(), 0, s>>>(a);
    } else {
        const unsigned blocks = (unsigned)((size_t)a.B * a.H + a.B);
        step_kernel<P, N, LM, false, 1><<<blocks, StepShape<P, N>::NTS + 64 * step_ring_waves<LM, false>(), 0, s>>>(a);
    }
    return hipGetLastError();
}

template <int P, int N>
static hipError_t launch_pn(const StepArgs &a, hipStream_t s) {
    if (a.L <= 16) return launch_lm<P, N, 16>(a, s);
    return launch_lm<P, N, kMaxRing>(a, s);
}

hipError_t launch_step(int P, int N, const StepArgs &a, hipStream_t s) {
    if (P == 16 && N == 16) return launch_pn<16, 16>(a, s);
    if (P == 64 && N == 64) return launch_pn<64, 64>(a, s);
    if (P == 64 && N == 128) return launch_pn<64, 128>(a, s);
    if (P == 128 && N == 128) return launch_pn<128, 128>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace replay
