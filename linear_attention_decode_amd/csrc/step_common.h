// step_common.h -- tiling, row copies and the bf16 ring wavefront shared by
// the fused step kernels (step.hip, step_copy.hip, verify_step.hip).
#pragma once
#include "ring_mx.h"

namespace replay {

template <int P, int N>
struct StepShape {
    static constexpr int VEC = 4;
    static constexpr int CHUNKS = P * N / VEC;
    // streaming threads: at most 8 chunks a lane (4096 chunks: 8 wavefronts)
    static constexpr int NTS = CHUNKS >= 4096 ? 512 : (CHUNKS < 256 ? CHUNKS : 256);
    static constexpr int ITER = CHUNKS / NTS;
    static constexpr int LPR = N / VEC;
    static constexpr int RPI = NTS / LPR;
    static_assert(CHUNKS % NTS == 0 && NTS % 64 == 0, "bad tiling");
    static_assert(LPR <= 64 && 64 % LPR == 0, "row group must sit in a wavefront");
};

// Raw 32-bit words of one io row (N elements), copied by the 64 lanes.
template <int N, bool IOB>
struct RowWords {
    static constexpr int WORDS = N * (IOB ? 2 : 4) / 4;
    static constexpr int WPL = (WORDS + 63) / 64;
    uint32_t w[WPL];
    __device__ __forceinline__ void load(const void *row, int lane) {
#pragma unroll
        for (int i = 0; i < WPL; ++i) {
            const int k = lane + 64 * i;
            w[i] = static_cast<const uint32_t *>(row)[k < WORDS ? k : WORDS - 1];
        }
    }
    __device__ __forceinline__ void store(void *row, int lane) const {
#pragma unroll
        for (int i = 0; i < WPL; ++i) {
            const int k = lane + 64 * i;
            if (k < WORDS) static_cast<uint32_t *>(row)[k] = w[i];
        }
    }
};

// The ring wavefronts for bf16 io: the same work with the output-only route
// on the matrix cores (ring_mx.h); wavefront rw covers entries 16rw..16rw+15
// (two wavefronts for a 32-entry ring).  Entry cold, this step's token, comes
// from the inputs (k row, query, v); the other operands from the ring, as in
// ring_wave_mx of the decode kernel, and every lane, clamped ones included,
// holds the values the decode kernel holds after an append, so the output
// of a non-folding step equals decode's bit for bit.  load() issues every
// load; finish() arrives and does the rest.  The token itself goes into the
// ring through the launch's writer workgroups (step_token_writer).
// A head of PROW rows can be split over workgroups: this one covers the P
// rows from p0 (its v values and its part of the ring term).
template <int P, int N, int LM, int PROW = P>
struct StepRingMx {
    using MX = MxRing<P, N, 1, LM>;
    static constexpr int VR = (P + 63) / 64;
    static constexpr uint32_t ES = 2;
    MX m;
    int p0;
    float a_in, dt_in, a_r, dt_r;
    RowWords<N, true> qrow;          // lane i: word i of the new q row
    uint32_t vin[MX::PW];            // the new v in the operand's pair layout (entry cold)
    static_assert(RowWords<N, true>::WPL == 1, "one word of a row per lane");

    __device__ __forceinline__ void load(const StepArgs &A, int lane, int rw, int b, int g, int h, size_t bh,
                                         int base, int cold, int p0_ = 0) {
        load_token(A, lane, b, g, bh, p0_);
        load_ring(A, lane, rw, b, g, bh, base, cold);
    }

    // this step's token: a, dt and the query row (none depends on the pointer)
    __device__ __forceinline__ void load_token(const StepArgs &A, int lane, int b, int g, size_t bh, int p0_ = 0) {
        p0 = p0_;
        a_in = A.a[bh];
        dt_in = A.dt[bh];
        qrow.load(static_cast<const char *>(A.q) + ((size_t)b * A.G + g) * N * ES, lane);
    }

    // the ring's entries (and this step's v row, which joins them as entry cold)
    __device__ __forceinline__ void load_ring(const StepArgs &A, int lane, int rw, int b, int g, size_t bh,
                                              int base, int cold) {
        const int L = A.L;
        const size_t gring = ((size_t)b * A.G + g) * L;
        const size_t hring = bh * L;
        const size_t gin = (size_t)b * A.G + g;
        const int bmod = base % L;
        auto slot = [&](int j) { return ring_slot(bmod, j, L); };
        const int lastr = cold > 0 ? cold - 1 : 0;   // clamp for ring loads (never used when cold == 0)
        const int lr = lane & 15, lq = lane >> 4;
        m.j0 = 16 * rw;
        const int sla = slot(lane < cold ? lane : lastr);
        a_r = A.ring_a[dta_index(b, bh, A.H, L, sla)];
        dt_r = A.ring_dt[dta_index(b, bh, A.H, L, sla)];
#pragma unroll
        for (int kb = 0; kb < MX::KB; ++kb) {
            const int c = MX::col(kb, lane);
            const int j = m.j0 + lr;   // entries < cold from the ring, the rest from this step's k
            const bool old = j < cold;
            m.ka[kb] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(old ? A.ring_k : A.k) +
                                                        (old ? (gring + slot(j)) * N : gin * N) + c);
        }
        const auto vres = make_rsrc(static_cast<const char *>(A.ring_v) + hring * PROW * ES, (uint32_t)(L * PROW * ES));
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int j = m.j0 + 4 * lq + kk;
            const uint32_t row = (uint32_t)slot(j < cold ? j : lastr) * PROW + p0;
#pragma unroll
            for (int pw = 0; pw < MX::PW; ++pw)
                m.vw[kk][pw] = __builtin_amdgcn_raw_buffer_load_b32(vres, (row + 2 * MX::vword(pw, lane)) * ES, 0, 0);
        }
#pragma unroll
        for (int pw = 0; pw < MX::PW; ++pw)
            vin[pw] = static_cast<const uint32_t *>(A.v)[(bh * PROW + p0) / 2 + MX::vword(pw, lane)];
    }

    // Returns this wavefront's arrival: the old count of its group counter.
    __device__ __forceinline__ int finish(const StepArgs &A, int lane, int b, int g, int cold, bool fold,
                                          float (*s_r)[P], float *s_abar, float (*s_U)[LM + 1], float (*s_K)[N],
                                          float (*s_sw)[LM]) {
        const int count = cold + 1;
        const int lr = lane & 15, lq = lane >> 4;
        int prev = -1;
        // Arrival of this ring wavefront (every ring wavefront arrives after
        // its own pointer read, which the loads above depend on).  Its result
        // is needed only at the very end.
        if (lane == 0) prev = atomicAdd(&A.sync[((size_t)b * (A.G + 1) + g) * kSyncStride], 1);

        // entry cold and past it: this step's token (the query, the B operand
        // of every column, gathered from the row's words)
#pragma unroll
        for (int kb = 0; kb < MX::KB; ++kb) {
            const int w0 = MX::col(kb, lane) / 2;
            m.qb[kb] = uint4{(uint32_t)__shfl((int)qrow.w[0], w0), (uint32_t)__shfl((int)qrow.w[0], w0 + 1),
                             (uint32_t)__shfl((int)qrow.w[0], w0 + 2), (uint32_t)__shfl((int)qrow.w[0], w0 + 3)};
        }
        m.aj = lane < cold ? a_r : (lane == cold ? a_in : 1.f);
        m.dtj = lane < cold ? dt_r : (lane == cold ? dt_in : 0.f);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int pw = 0; pw < MX::PW; ++pw)
                if (m.j0 + 4 * lq + kk >= cold) m.vw[kk][pw] = vin[pw];

        if (!fold) {
            const f32x4 dk = m.dots(lane);
            m.weights(lane, count, s_abar, s_sw);
            m.term(lane, dk, s_r, s_sw);
        } else {
            // state-and-output route: stage U[p][j] = s_j v_j[p] and K[j][n] = k_j[n]
            // for this wavefront's entries
            m.weights(lane, count, s_abar, s_sw);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int j = m.j0 + 4 * lq + kk;
                if (j < count) {
                    const float sj = s_sw[0][j];
#pragma unroll
                    for (int pw = 0; pw < MX::PW; ++pw)
#pragma unroll
                        for (int half = 0; half < 2; ++half) {
                            const int p = 32 * pw + 2 * lr + half;
                            if (p < P) s_U[p][j] = sj * MX::vval(m.vw[kk][pw], half);
                        }
                }
            }
            const int j = m.j0 + lr;
            if (j < count) {
#pragma unroll
                for (int kb = 0; kb < MX::KB; ++kb) {
                    const int c = 32 * kb + 8 * lq;
                    if (c < N) {
                        IoVec<true, 8> kv;
                        kv.r = m.ka[kb];
                        float kk8[8];
                        kv.widen(kk8);
#pragma unroll
                        for (int e = 0; e < 8; ++e) s_K[j][c + e] = kk8[e];
                    }
                }
            }
        }
        return prev;
    }
};

// Arrival at a sequence's counter: its G groups and its writer workgroup
// arrive there; the last moves the pointer (every workgroup of the sequence
// has read it by then).
__device__ __forceinline__ void step_seq_arrive(const StepArgs &A, int b, int pos, bool fold) {
    int32_t *seq = A.sync + ((size_t)b * (A.G + 1) + A.G) * kSyncStride;
    if (atomicAdd(seq, 1) == A.G) {
        atomicExch(seq, 0);
        A.pos[b] = pos + 1;
        if (fold) A.base[b] = pos + 1;
    }
}

// The writer workgroup of sequence b: this step's token (the v row, dt and
// a of every head, the q and k rows of every group) goes into ring slot
// pos mod L, which no workgroup of this launch reads (entries < count - 1
// only).  Writers follow every compute workgroup in the grid, so their
// stores land in the launch's tail instead of between the tile reads.
// FOLDS: the launch folds rings with count >= flush_at (base moves too).
template <int PH, int N, bool IOB, bool FOLDS>
__device__ __forceinline__ void step_token_writer(const StepArgs &A, int b, int tid, int nt) {
    const int L = A.L, H = A.H, G = A.G;
    const int base = A.base[b], pos = A.pos[b];
    const int cold = pos - base;
    if (cold + 1 > L || pos == 2147483647) return;   // left unchanged; the compute workgroups report it
    const int sn = ring_slot(base % L, cold, L);
    constexpr int ES = IOB ? 2 : 4;
    constexpr int VP = PH * ES / 16;   // 16-byte pieces of a v row
    constexpr int KP = N * ES / 16;    // of a q or k row
    static_assert(PH * ES % 16 == 0 && N * ES % 16 == 0, "rows of whole 16-byte pieces");
    for (int i = tid; i < H * VP; i += nt) {
        const size_t bh = (size_t)b * H + i / VP;
        const uint4 x = reinterpret_cast<const uint4 *>(static_cast<const char *>(A.v) + bh * PH * ES)[i % VP];
        reinterpret_cast<uint4 *>(static_cast<char *>(A.ring_v) + (bh * L + sn) * PH * ES)[i % VP] = x;
    }
    for (int i = tid; i < 2 * G * KP; i += nt) {
        const int r = i % (G * KP);
        const size_t gi = (size_t)b * G + r / KP;
        const bool kr = i >= G * KP;
        const uint4 x = reinterpret_cast<const uint4 *>(static_cast<const char *>(kr ? A.k : A.q) + gi * N * ES)[r % KP];
        reinterpret_cast<uint4 *>(static_cast<char *>(kr ? A.ring_k : A.ring_q) + (gi * L + sn) * N * ES)[r % KP] = x;
    }
    for (int i = tid; i < H; i += nt) {
        const size_t bh = (size_t)b * H + i;
        A.ring_dt[dta_index(b, bh, H, L, sn)] = A.dt[bh];
        A.ring_a[dta_index(b, bh, H, L, sn)] = A.a[bh];
    }
    __syncthreads();   // every wavefront of the workgroup has read the pointer
    if (tid == 0) {
        const int need = A.flush_at > 1 ? A.flush_at : 1;
        step_seq_arrive(A, b, pos, FOLDS && cold + 1 >= need);
    }
}

}  // namespace replay
