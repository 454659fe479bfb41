// flush.hip -- rank-c checkpoint update and low-precision copy for gfx950.
//
// For every (sequence, head) whose ring holds c >= max(min_count, 1) entries:
//     S0 <- abar_c S0 + sum_{j=1..c} s_{j,c} v_j k_j^T
// (page "ReplaySSM: Cachear Inputs, No Estado", section "Los dos caminos",
// eq. "Ruta estado y salida"; "Decodificacion estandar", step 4: the
// buffer is folded into the checkpoint and written once), with
// abar_c = prod_{m<=c} a_m and s_{j,c} = dt_j prod_{j<m<=c} a_m.  The fold
// reads the float32 master (or, for a checkpoint load, a float32 source with
// an empty ring) and writes the float32 master and/or a bf16 / e4m3 / MX FP4
// copy (page "ReplaySSM: Cache SSM Inputs, Not State", Abstract: a
// low-precision copy serves outputs, a higher-precision checkpoint takes the
// updates).  e4m3 copies carry one scale per head: scale = amax/448 (1 if
// amax = 0), code = e4m3(x / scale), round to nearest even, saturating.  A
// shared low-precision checkpoint (no master) folds in flush_shared.hip.
//
// HC heads per workgroup.  The tile streams through registers (16-byte
// master chunks); s_j v_j (P x c) and k_j (c x N) are staged in LDS, so each
// state element costs c FMAs against two LDS broadcasts per ring entry.  The
// last workgroup of a sequence to arrive at its counter moves the base
// pointer, once every workgroup of the sequence has read it.
#include "device_common.h"

namespace replay {

template <int P, int N>
struct FlushShape {
    static constexpr int VEC = 4;
    static constexpr int CHUNKS = P * N / VEC;
    static constexpr int NT = CHUNKS < 256 ? CHUNKS : 256;
    static constexpr int ITER = CHUNKS / NT;
    static constexpr int LPR = N / VEC;
    static constexpr int RPI = NT / LPR;
    static_assert(CHUNKS % NT == 0 && NT % 64 == 0, "bad tiling");
    static_assert(LPR <= 64 && 64 % LPR == 0, "row group must sit in a wavefront");
};

// HC heads of one group per workgroup, pipelined (each head's loads are
// issued before the previous head is folded; the group's k rows are staged
// once): a flush that finds nothing due costs B*H/HC workgroups that only
// read the pointer.
template <int P, int N, int COPY, bool WRITE_MASTER, bool IOB, int HC>
__global__ __launch_bounds__((FlushShape<P, N>::NT)) void flush_kernel(FlushArgs args) {
    using Sh = FlushShape<P, N>;
    constexpr int VEC = Sh::VEC, NT = Sh::NT, ITER = Sh::ITER, LPR = Sh::LPR, RPI = Sh::RPI;

    extern __shared__ __align__(16) float smem[];   // U [P][c] then K [c][N]
    __shared__ float s_a[kMaxRing], s_dt[kMaxRing], s_w[kMaxRing];
    __shared__ float s_abar;
    __shared__ float s_red[NT / 64];

    constexpr int JG = NT / P;                      // thread groups over ring entries
    constexpr int JPG = (kMaxRing + JG - 1) / JG;   // v values per thread
    constexpr int KPT = (kMaxRing * (N / 4) + NT - 1) / NT;   // k pieces per thread
    static_assert(NT % P == 0, "ring groups");

    const RingView &r = args.r;
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int HW = r.H / HC;
    const int b = lid / HW, h0 = (lid % HW) * HC;
    const int g = (h0 * r.G) / r.H;   // the HC heads share this group
    const int tid = threadIdx.x, lane = tid & 63;
    const int L = r.L;

    const int base = r.base[b];
    const int pos = r.pos[b];
    int count = 0;
    if (!args.force_empty) {
        count = pos - base;
        const int need = args.min_count > 1 ? args.min_count : 1;
        if (count < need) return;  // uniform: nothing to fold for this sequence
    }
    // Every wavefront arrives at its group's counter right after its own
    // pointer read (the counter expects one arrival per wavefront), so no
    // wavefront can read a base the sequence's last arrival has moved; that
    // last arrival moves base at its very end.
    int prev = -1;
    if (lane == 0) prev = atomicAdd(&args.sync[((size_t)b * (r.G + 1) + g) * kSyncStride], 1);

    const int bmod = base % L;
    auto slot = [&](int j) { return ring_slot(bmod, j, L); };   // entry j (0-based) of the ring
    const size_t gring = ((size_t)b * r.G + g) * L;
    const int last = count > 0 ? count - 1 : 0;   // clamp for ring loads (clamped values are never used)
    const int vp = tid % P, vg = tid / P;

    // What one head needs from memory: its tile and its ring entries (a, dt,
    // v).  The HC heads of a workgroup are pipelined: head hl+1's loads are
    // issued before head hl is folded, so the memory latency is paid once per
    // workgroup instead of once per head.
    struct HeadLoads {
        Chunk<ST_F32, VEC> ch[ITER];
        float a, dt;
        IoVec<IOB, 1> v[JPG];
    };
    auto issue = [&](int hl, HeadLoads &hd) {
        const size_t bh = (size_t)b * r.H + h0 + hl;
        const size_t tile = bh * (size_t)(P * N);
#pragma unroll
        for (int i = 0; i < ITER; ++i) hd.ch[i].load(args.S_in, tile + (size_t)(i * NT + tid) * VEC);
        hd.a = 1.f;
        hd.dt = 0.f;
        if (count > 0) {
            const size_t hring = bh * L;
            const int sl = slot(tid < count ? tid : last);
            hd.a = r.a[dta_index(b, bh, r.H, L, sl)];
            hd.dt = r.dt[dta_index(b, bh, r.H, L, sl)];
#pragma unroll
            for (int i = 0; i < JPG; ++i) {
                const int j = vg + i * JG;
                hd.v[i].load(r.v, (hring + slot(j < count ? j : last)) * P + vp);
            }
        }
    };

    // 1. the first head's loads, then the group's k rows (shared by the HC
    // heads: loaded and staged once)
    HeadLoads cur, nxt;
    issue(0, cur);
    IoVec<IOB, 4> kraw[KPT];
    if (count > 0) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int piece = tid + i * NT;
            const int j = piece / (N / 4), n = (piece % (N / 4)) * 4;
            kraw[i].load(r.k, (gring + slot(j < count ? j : last)) * N + n);
        }
    }
    float *U = smem;
    float *Ks = smem + P * count;

#pragma unroll
    for (int hl = 0; hl < HC; ++hl) {
    const size_t bh = (size_t)b * r.H + h0 + hl;
    const size_t tile = bh * (size_t)(P * N);
    if (hl + 1 < HC) issue(hl + 1, nxt);

    // 2. segment weights of the c entries
    if (tid < count) {
        s_a[tid] = cur.a;
        s_dt[tid] = cur.dt;
    }
    __syncthreads();
    if (tid < count) {
        float s = s_dt[tid];
        for (int m = tid + 1; m < count; ++m) s *= s_a[m];
        s_w[tid] = s;
    }
    if (tid == 0) {
        float ab = 1.f;
        for (int m = 0; m < count; ++m) ab *= s_a[m];
        s_abar = ab;
    }
    __syncthreads();

    // 3. stage U[p][j] = s_j v_j[p] (and, for the first head, K[j][n] = k_j[n])
#pragma unroll
    for (int i = 0; i < JPG; ++i) {
        const int j = vg + i * JG;
        if (j < count) U[vp * count + j] = s_w[j] * cur.v[i].value();
    }
    if (hl == 0) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int piece = tid + i * NT;
            const int j = piece / (N / 4), n = (piece % (N / 4)) * 4;
            if (j < count) {
                float kk[4];
                kraw[i].widen(kk);
#pragma unroll
                for (int e = 0; e < 4; ++e) Ks[j * N + n + e] = kk[e];
            }
        }
    }
    __syncthreads();

    // 4. x = abar * S0 + sum_j U[row][j] K[j][col]
    const float abar = s_abar;
    const int col0 = (tid % LPR) * VEC;
    float x[ITER][VEC];
#pragma unroll
    for (int i = 0; i < ITER; ++i) {
        cur.ch[i].widen(x[i], 1.0f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[i][e] *= abar;
    }
    for (int j = 0; j < count; ++j) {
        const f32x4 kk = *reinterpret_cast<const f32x4 *>(&Ks[j * N + col0]);
#pragma unroll
        for (int i = 0; i < ITER; ++i) {
            const int row = i * RPI + tid / LPR;
            const float u = U[row * count + j];
            x[i][0] = fmaf(u, kk.x, x[i][0]);
            x[i][1] = fmaf(u, kk.y, x[i][1]);
            x[i][2] = fmaf(u, kk.z, x[i][2]);
            x[i][3] = fmaf(u, kk.w, x[i][3]);
        }
    }

    // 5. float32 master
    if constexpr (WRITE_MASTER) {
#pragma unroll
        for (int i = 0; i < ITER; ++i) {
            f32x4 o = {x[i][0], x[i][1], x[i][2], x[i][3]};
            __builtin_nontemporal_store(o, reinterpret_cast<f32x4 *>(args.S_out + tile + (size_t)(i * NT + tid) * VEC));
        }
    }

    // 6. low-precision copy
    if constexpr (COPY == ST_BF16) {
        uint16_t *cp = static_cast<uint16_t *>(args.copy_out) + tile;
#pragma unroll
        for (int i = 0; i < ITER; ++i) {
            u32x2 o;
            o.x = f32x2_to_bf16_pair(x[i][0], x[i][1]);
            o.y = f32x2_to_bf16_pair(x[i][2], x[i][3]);
            __builtin_nontemporal_store(o, reinterpret_cast<u32x2 *>(cp + (size_t)(i * NT + tid) * VEC));
        }
    } else if constexpr (COPY == ST_FP8) {
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < ITER; ++i)
#pragma unroll
            for (int e = 0; e < VEC; ++e) amax = fmaxf(amax, fabsf(x[i][e]));
#pragma unroll
        for (int bit = 5; bit >= 0; --bit) amax = fmaxf(amax, lane_partner(amax, bit));
        if (lane == 0) s_red[tid / 64] = amax;
        __syncthreads();
        amax = s_red[0];
#pragma unroll
        for (int i = 1; i < NT / 64; ++i) amax = fmaxf(amax, s_red[i]);
        const float sig = amax > 0.f ? amax / 448.0f : 1.0f;   // correctly rounded divide
        const ScaleDiv dv(sig);
        uint8_t *cp = static_cast<uint8_t *>(args.copy_out) + tile;
        dv.run([&](auto div) {
#pragma unroll
            for (int i = 0; i < ITER; ++i) {
                const uint32_t o = f32x4_to_fp8(div(x[i][0]), div(x[i][1]), div(x[i][2]), div(x[i][3]));
                __builtin_nontemporal_store(o, reinterpret_cast<uint32_t *>(cp + (size_t)(i * NT + tid) * VEC));
            }
        });
        if (tid == 0) static_cast<float *>(args.scale_out)[bh] = sig;
    } else if constexpr (COPY == ST_FP4) {
        // MX FP4: the 32 consecutive values of 8 neighbouring lanes share the
        // scale X = 2^(floor(log2 amax) - 2); codes are e2m1(x / X), the
        // division exact (ldexp), converted by the hardware (nearest even,
        // saturating at 6); first value of a pair in the low nibble
        uint8_t *cp = static_cast<uint8_t *>(args.copy_out);
        uint8_t *scl = static_cast<uint8_t *>(args.scale_out);
#pragma unroll
        for (int i = 0; i < ITER; ++i) {
            float amax = fmaxf(fmaxf(fabsf(x[i][0]), fabsf(x[i][1])), fmaxf(fabsf(x[i][2]), fabsf(x[i][3])));
#pragma unroll
            for (int bit = 2; bit >= 0; --bit) amax = fmaxf(amax, lane_partner(amax, bit));
            const int se = mxfp4_block_exp(amax);
            const size_t e0 = tile + (size_t)(i * NT + tid) * VEC;
            *reinterpret_cast<uint16_t *>(cp + e0 / 2) = mxfp4_codes4(x[i][0], x[i][1], x[i][2], x[i][3], se);
            if ((tid & 7) == 0) scl[e0 / 32] = (uint8_t)(se + 127);
        }
    }

    if (hl + 1 < HC) {
        __syncthreads();   // LDS is reused by the next head
        cur = nxt;
    }
    }

    // Last wavefront of its group: the group arrives at the sequence's
    // counter; the last group means every wavefront of the sequence has read base.
    if (lane == 0 && prev == r.H / r.G / HC * (NT / 64) - 1) {
        int32_t *seq = args.sync + (size_t)b * (r.G + 1) * kSyncStride;
        atomicExch(seq + (size_t)g * kSyncStride, 0);
        if (atomicAdd(seq + (size_t)r.G * kSyncStride, 1) == r.G - 1) {
            atomicExch(seq + (size_t)r.G * kSyncStride, 0);
            args.base_out[b] = pos;
        }
    }
}

template <int P, int N, int COPY, bool WM, int HC>
static hipError_t launch_hc(const FlushArgs &a, hipStream_t s) {
    using Sh = FlushShape<P, N>;
    const unsigned blocks = (unsigned)((size_t)a.r.B * a.r.H / HC);
    const size_t lds = (size_t)(P + N) * a.r.L * sizeof(float);
    if (a.r.io_bf16)
        flush_kernel<P, N, COPY, WM, true, HC><<<blocks, Sh::NT, lds, s>>>(a);
    else
        flush_kernel<P, N, COPY, WM, false, HC><<<blocks, Sh::NT, lds, s>>>(a);
    return hipGetLastError();
}

// Four heads per workgroup only for flushes that fold full rings only
// (min_count >= L): in the standard schedule those find nothing due on all
// but one step in L, where the smaller grid saves most; a flush that folds
// part of the batch every call (speculative rounds) and a checkpoint load
// keep one head per workgroup, which folds faster.
template <int P, int N, int COPY, bool WM>
static hipError_t launch_one(const FlushArgs &a, hipStream_t s) {
    constexpr int HC = 4;
    if (!a.force_empty && a.min_count >= a.r.L && (a.r.H / a.r.G) % HC == 0)
        return launch_hc<P, N, COPY, WM, HC>(a, s);
    return launch_hc<P, N, COPY, WM, 1>(a, s);
}

template <int P, int N>
static hipError_t launch_pn(int st_in, int st_copy, bool wm, const FlushArgs &a, hipStream_t s) {
    if (st_in == ST_F32 && wm) {           // separated: the float32 master takes the update
        if (st_copy == ST_BF16) return launch_one<P, N, ST_BF16, true>(a, s);
        if (st_copy == ST_FP8) return launch_one<P, N, ST_FP8, true>(a, s);
        if (st_copy == ST_FP4) return launch_one<P, N, ST_FP4, true>(a, s);
        return launch_one<P, N, -1, true>(a, s);
    }
    if (st_in == ST_F32) {                 // shared mode, loading a float32 checkpoint
        if (st_copy == ST_BF16) return launch_one<P, N, ST_BF16, false>(a, s);
        if (st_copy == ST_FP8) return launch_one<P, N, ST_FP8, false>(a, s);
        if (st_copy == ST_FP4) return launch_one<P, N, ST_FP4, false>(a, s);
        return hipErrorInvalidValue;
    }
    if (wm || a.force_empty) return hipErrorInvalidValue;   // shared mode: the copy is the only checkpoint
    if (st_in == st_copy) return launch_flush_shared(P, N, st_in, a, s);   // flush_shared.hip
    return hipErrorInvalidValue;
}

hipError_t launch_flush(int P, int N, int st_in, int st_copy, bool write_master, const FlushArgs &a,
                        hipStream_t s) {
    if (P == 16 && N == 16) return launch_pn<16, 16>(st_in, st_copy, write_master, a, s);
    if (P == 64 && N == 64) return launch_pn<64, 64>(st_in, st_copy, write_master, a, s);
    if (P == 64 && N == 128) return launch_pn<64, 128>(st_in, st_copy, write_master, a, s);
    if (P == 128 && N == 128) return launch_pn<128, 128>(st_in, st_copy, write_master, a, s);
    return hipErrorInvalidValue;
}

}  // namespace replay
