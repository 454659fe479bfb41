// flush_shared.hip -- the fold of a shared low-precision checkpoint (bf16,
// e4m3 or MX FP4 copy, no float32 master) on the matrix cores, for gfx950.
//
// For every (sequence, head) whose ring holds c >= max(min_count, 1) entries:
//     S0 <- abar_c deQ(S0) + sum_{j=1..c} s_{j,c} v_j k_j^T,   then S0 <- Q(S0)
// (page "ReplaySSM: Cachear Inputs, No Estado", section "Los dos caminos",
// eq. "Ruta estado y salida"; page "ReplaySSM: Cache SSM Inputs, Not State",
// Abstract: the low-precision state is the checkpoint), with the flush
// kernel's segment weights and the same quantisers (e4m3: per-head scale
// amax/448, codes e4m3(x / scale) with a correctly rounded division; FP4: MX
// blocks of 32 with E8M0 scales; bf16: round to nearest even).  Built with
// MFMA results kept in VGPRs (-amdgpu-mfma-vgpr-form): with accumulators in
// AGPRs every product paid two copies per element.
#include <type_traits>

#include "device_common.h"

namespace replay {

// Views of the staging buffer at the widths it is written and read with.  A
// wavefront writes it at one width and reads it back at another with no
// barrier in between, so the accesses must not be taken as unrelated by type
// (type-based alias analysis would let the compiler reorder a 4-byte store
// past a 16-byte load of the same bytes): may_alias keeps program order.
typedef uint16_t lds_u16 __attribute__((may_alias));
typedef uint32_t lds_u32 __attribute__((may_alias));
typedef uint32_t lds_u32x2 __attribute__((ext_vector_type(2), may_alias));
typedef uint32_t lds_u32x4 __attribute__((ext_vector_type(4), may_alias));

// Shared low-precision checkpoint (the copy is the only state): the fold on
// the matrix cores.  At 1 or 2 bytes an element the rank-c update costs
// 2c flops per element, 16 to 32 per byte moved at c = 16: more than the
// float32 vector units (no packed operations) sustain at HBM speed, while
// v_mfma_f32_16x16x4_f32 forms it at twice their rate.  Wavefront w owns rows
// 16w..16w+15 of one head's tile; column tile nt is the 16 x 16 product
//     D[n][p] = abar S0[p][n] + sum_j K[j][n] U[p][j],  K[j][n] = k_j[n], U[p][j] = s_j v_j[p]
// (A = K^T: lane (lr, lg) of k-step s gives k_{4s+lg}[16nt + lr]; B = U^T:
// U[16w + lr][4s + lg]), so lane (lr, lg) holds columns 16nt + 4lg .. +3
// of row 16w + lr.  All L_max / 4 k-steps run; entry slots past the count
// have weight 0 and zero K rows.
// Rows of 64 or more columns go between HBM and that layout through the
// wavefront's own LDS buffer (16-byte runs along the rows both ways: read
// in the layout itself, every instruction would touch 16 rows in pieces of
// 2 to 8 bytes); 16-column rows are already contiguous in it.
template <int P, int N, int ST>
struct SharedFoldShape {
    static constexpr int NW = P / 16, NT = 64 * NW, NTL = N / 16;   // wavefronts, threads, column tiles
    static constexpr int RB = ST == ST_FP4 ? N / 2 : (ST == ST_FP8 ? N : 2 * N);   // bytes of a row
    static constexpr int CB = ST == ST_FP4 ? 2 : (ST == ST_FP8 ? 4 : 8);          // bytes of a lane's chunk
    static constexpr bool STAGE = N >= 64;
    static constexpr int TROW = RB + 16;                          // staging row stride, bytes
    static constexpr int C16 = 16 * RB / 16;                      // 16-byte runs of a wavefront's rows
    static constexpr int RI = (C16 + 63) / 64;                    // runs per lane
    static_assert(!STAGE || RB % 16 == 0, "rows of whole 16-byte runs");
};

template <int P, int N, int ST, bool IOB, int LM, int HC>
__global__ __launch_bounds__(P / 16 * 64) void flush_shared_kernel(FlushArgs args) {
    using SF = SharedFoldShape<P, N, ST>;
    constexpr int NW = SF::NW, NT = SF::NT, NTL = SF::NTL, RB = SF::RB, CB = SF::CB, RI = SF::RI;
    constexpr int KS = LM / 4;                                  // k-steps: every entry slot of the ring
    constexpr int SKS = N % 64 == 0 ? N + 16 : N;               // LDS row stride of K (the 4 lane groups' rows
                                                                // fall in different banks)
    constexpr int KPT = (LM * (N / 4) + NT - 1) / NT;           // k pieces (4 values) per thread
    static_assert(LM <= 64 && HC <= NW, "wavefront w < HC forms head w's weights, one lane per entry");
    __shared__ float s_w[HC][LM];
    __shared__ float s_abar[HC];
    __shared__ float s_red[HC][NW];
    __shared__ __align__(16) float s_K[LM][SKS];
    __shared__ __align__(16) uint8_t s_T[SF::STAGE ? NW : 1][SF::STAGE ? 16 : 1][SF::STAGE ? SF::TROW : 16];

    const RingView &r = args.r;
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int HW = r.H / HC;
    const int b = lid / HW, h0 = (lid % HW) * HC;
    const int g = (h0 * r.G) / r.H;   // the HC heads share this group
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int L = r.L;

    const int base = r.base[b];
    const int pos = r.pos[b];
    const int count = pos - base;
    if (count < (args.min_count > 1 ? args.min_count : 1)) return;   // uniform: nothing to fold
    // every wavefront arrives at its group's counter right after its own
    // pointer read (one arrival per wavefront)
    int prev = -1;
    if (lane == 0) prev = atomicAdd(&args.sync[((size_t)b * (r.G + 1) + g) * kSyncStride], 1);

    const int p = 16 * wave + lr;
    const int bmod = base % L;
    auto slot = [&](int j) { return ring_slot(bmod, j, L); };
    const int last = count - 1;
    const size_t gring = ((size_t)b * r.G + g) * L;
    auto run_row = [&](int c) { return c / (RB / 16); };
    auto run_col = [&](int c) { return 16 * (c % (RB / 16)); };

    // What one head needs from memory: the copy's rows of this wavefront
    // (16-byte runs, or the chunks themselves for 16-column rows), their
    // scales, and the v values of its k-steps.  Every head's loads are
    // issued before the first is folded: one memory latency per workgroup.
    struct HeadLoads {
        u32x4 run[SF::STAGE ? RI : 1];
        Chunk<ST, 4> ch[SF::STAGE ? 1 : NTL];
        int se[ST == ST_FP4 && SF::STAGE ? NTL : 1];
        float sc;
        IoVec<IOB, 1> vv[KS];
    };
    auto issue = [&](int hl, HeadLoads &hd) {
        const size_t bh = (size_t)b * r.H + h0 + hl;
        const size_t tile = bh * (size_t)(P * N);
        const size_t rowe = tile + (size_t)p * N + 4 * lg;
        if constexpr (SF::STAGE) {
            const uint8_t *src = static_cast<const uint8_t *>(args.S_in) + (tile + (size_t)16 * wave * N) * RB / N;
#pragma unroll
            for (int i = 0; i < RI; ++i) {
                const int c = lane + 64 * i;
                if (c < SF::C16)
                    hd.run[i] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4 *>(src + (size_t)run_row(c) * RB + run_col(c)));
            }
            if constexpr (ST == ST_FP4) {
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt)
                    hd.se[nt] = (int)static_cast<const uint8_t *>(args.scale_in)[(rowe + 16 * nt) / 32] - 127;
            }
        } else {
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                if constexpr (ST == ST_FP4)
                    hd.ch[nt].load_mx(args.S_in, args.scale_in, rowe + 16 * nt);
                else
                    hd.ch[nt].load(args.S_in, rowe + 16 * nt);
            }
        }
        hd.sc = (ST == ST_FP8) ? static_cast<const float *>(args.scale_in)[bh] : 1.0f;
        const size_t hring = bh * L;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int j = 4 * s + lg;
            hd.vv[s].load(r.v, (hring + slot(j < count ? j : last)) * P + p);
        }
    };

    // 1. the heads' loads, the entries' a and dt (wavefront w < HC: head
    // h0 + w), the group's k rows (shared by the HC heads)
    HeadLoads hd[HC];
#pragma unroll
    for (int hl = 0; hl < HC; ++hl) issue(hl, hd[hl]);
    float aj = 1.f, dtj = 0.f;
    if (wave < HC && lane < count) {
        const size_t bhw = (size_t)b * r.H + h0 + wave;
        aj = r.a[dta_index(b, bhw, r.H, L, slot(lane))];
        dtj = r.dt[dta_index(b, bhw, r.H, L, slot(lane))];
    }
    IoVec<IOB, 4> kraw[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int piece = tid + i * NT;
        const int j = piece / (N / 4), n = (piece % (N / 4)) * 4;
        if (j < count) kraw[i].load(r.k, (gring + slot(j)) * N + n);
    }

    // 2. K staged as float32 (rows past the count as zeros: every k-step
    // runs, and a dead entry's products are 0 * 0); segment weights
    // (wavefront w, lane j, head h0 + w: the same left-to-right products as
    // the vector fold, factors broadcast from the lanes that hold them)
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int piece = tid + i * NT;
        const int j = piece / (N / 4), n = (piece % (N / 4)) * 4;
        if (j < LM) {
            float kk[4] = {0.f, 0.f, 0.f, 0.f};
            if (j < count) kraw[i].widen(kk);
            *reinterpret_cast<f32x4 *>(&s_K[j][n]) = f32x4{kk[0], kk[1], kk[2], kk[3]};
        }
    }
    if (wave < HC) {
        float prod = dtj, run = 1.f;
#pragma unroll
        for (int m = 0; m < LM; ++m) {
            if (m < count) {
                const float am = bcast(aj, m);
                if (m > lane) prod *= am;
                run *= am;
            }
        }
        if (lane < LM) s_w[wave][lane] = lane < count ? prod : 0.f;
        if (lane == 0) s_abar[wave] = run;
    }
    // LDS-only barrier: the arrival atomic need not have returned
    lds_barrier();

#pragma unroll
    for (int hl = 0; hl < HC; ++hl) {
        const size_t bh = (size_t)b * r.H + h0 + hl;
        const size_t tile = bh * (size_t)(P * N);
        const size_t rowe = tile + (size_t)p * N + 4 * lg;   // element of this lane's chunk in column tile 0
        const size_t wbytes = (tile + (size_t)16 * wave * N) * RB / N;   // this wavefront's rows, as bytes
        const HeadLoads &cur = hd[hl];

        // 3. the rows into the operand layout through this wavefront's own
        // buffer (every lane's accesses on one side of each wave_lds_sync:
        // the previous head's read-back is done before these writes, these
        // writes before the reads), then D = abar S0 + K^T U^T, tile by tile
        Chunk<ST, 4> ch[NTL];
        if constexpr (SF::STAGE) {
            if (hl > 0) wave_lds_sync();
#pragma unroll
            for (int i = 0; i < RI; ++i) {
                const int c = lane + 64 * i;
                if (c < SF::C16) *reinterpret_cast<lds_u32x4 *>(&s_T[wave][run_row(c)][run_col(c)]) = cur.run[i];
            }
            wave_lds_sync();
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                const uint8_t *t = &s_T[wave][lr][(16 * nt + 4 * lg) * CB / 4];
                if constexpr (ST == ST_BF16) {
                    const lds_u32x2 u = *reinterpret_cast<const lds_u32x2 *>(t);
                    ch[nt].raw[0] = u.x;
                    ch[nt].raw[1] = u.y;
                } else if constexpr (ST == ST_FP8) {
                    ch[nt].raw[0] = *reinterpret_cast<const lds_u32 *>(t);
                } else {
                    ch[nt].raw[0] = *reinterpret_cast<const lds_u16 *>(t);
                    ch[nt].se = cur.se[nt];
                }
            }
        } else {
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) ch[nt] = cur.ch[nt];
        }
        // S0 abar = code * (scale abar): one product an element (FP4: the
        // block's power of two joins abar exactly)
        const float abar = s_abar[hl];
        f32x4 acc[NTL];
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) {
            float x[4];
            ch[nt].widen(x, 1.0f);
            float f = abar;
            if constexpr (ST == ST_FP8) f = cur.sc * abar;
            if constexpr (ST == ST_FP4) f = ldexpf(abar, ch[nt].se);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[nt][e] = x[e] * f;
        }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int j = 4 * s + lg;
            const float bu = s_w[hl][j] * cur.vv[s].value();
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt)
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(s_K[j][16 * nt + lr], bu, acc[nt], 0, 0, 0);
        }

        // 4. the new copy: codes per chunk, then out in place (16-byte runs
        // through the staging buffer, or the chunks for 16-column rows)
        uint32_t code[NTL][CB >= 4 ? CB / 4 : 1];
        if constexpr (ST == ST_BF16) {
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                code[nt][0] = f32x2_to_bf16_pair(acc[nt][0], acc[nt][1]);
                code[nt][1] = f32x2_to_bf16_pair(acc[nt][2], acc[nt][3]);
            }
        } else if constexpr (ST == ST_FP8) {
            float amax = 0.f;
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(acc[nt][e]));
#pragma unroll
            for (int bit = 5; bit >= 0; --bit) amax = fmaxf(amax, lane_partner(amax, bit));
            if (lane == 0) s_red[hl][wave] = amax;
            lds_barrier();
            amax = s_red[hl][0];
#pragma unroll
            for (int i = 1; i < NW; ++i) amax = fmaxf(amax, s_red[hl][i]);
            const float sig = amax > 0.f ? amax / 448.0f : 1.0f;   // correctly rounded divide
            const ScaleDiv dv(sig);
            dv.run([&](auto div) {
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt)
                    code[nt][0] = f32x4_to_fp8(div(acc[nt][0]), div(acc[nt][1]), div(acc[nt][2]), div(acc[nt][3]));
            });
            if (tid == 0) static_cast<float *>(args.scale_out)[bh] = sig;
        } else {
            // MX FP4: a block is 32 consecutive values of the row-major tile --
            // column tiles 2bb and 2bb+1 of one row (N >= 32: lanes lr + 16 lg),
            // or rows p, p+1 of the single column tile (N = 16: lanes lr, lr ^ 1
            // and their groups); the lane of the block's first value writes its scale
            uint8_t *scl = static_cast<uint8_t *>(args.scale_out);
            constexpr int TPB = N >= 32 ? 2 : 1;   // column tiles per block
#pragma unroll
            for (int bb = 0; bb < NTL / TPB; ++bb) {
                float amax = 0.f;
#pragma unroll
                for (int t = 0; t < TPB; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(acc[TPB * bb + t][e]));
                amax = fmaxf(amax, lane_partner(amax, 5));
                amax = fmaxf(amax, lane_partner(amax, 4));
                if constexpr (N < 32) amax = fmaxf(amax, lane_partner(amax, 0));
                const int se = mxfp4_block_exp(amax);
#pragma unroll
                for (int t = 0; t < TPB; ++t) {
                    const f32x4 x = acc[TPB * bb + t];
                    code[TPB * bb + t][0] = mxfp4_codes4(x[0], x[1], x[2], x[3], se);
                }
                const bool first = lg == 0 && (N >= 32 || (lr & 1) == 0);
                if (first) scl[(rowe + 16 * TPB * bb) / 32] = (uint8_t)(se + 127);
            }
        }
        if constexpr (SF::STAGE) {
            // the buffer still holds this wavefront's old rows, all read above
            // (the quantisation's divergent branches may sit in between: the
            // codes of every lane are in before any lane reads a run back)
            wave_lds_sync();
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                uint8_t *t = &s_T[wave][lr][(16 * nt + 4 * lg) * CB / 4];
                if constexpr (ST == ST_BF16)
                    *reinterpret_cast<lds_u32x2 *>(t) = lds_u32x2{code[nt][0], code[nt][1]};
                else if constexpr (ST == ST_FP8)
                    *reinterpret_cast<lds_u32 *>(t) = code[nt][0];
                else
                    *reinterpret_cast<lds_u16 *>(t) = (uint16_t)code[nt][0];
            }
            uint8_t *dst = static_cast<uint8_t *>(args.copy_out) + wbytes;
            wave_lds_sync();
#pragma unroll
            for (int i = 0; i < RI; ++i) {
                const int c = lane + 64 * i;
                if (c < SF::C16)
                    __builtin_nontemporal_store(u32x4(*reinterpret_cast<const lds_u32x4 *>(&s_T[wave][run_row(c)][run_col(c)])),
                                                reinterpret_cast<u32x4 *>(dst + (size_t)run_row(c) * RB + run_col(c)));
            }
        } else {
            uint8_t *cp = static_cast<uint8_t *>(args.copy_out);
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                const size_t byte = (rowe + 16 * nt) * CB / 4;
                if constexpr (ST == ST_BF16)
                    __builtin_nontemporal_store(u32x2{code[nt][0], code[nt][1]}, reinterpret_cast<u32x2 *>(cp + byte));
                else if constexpr (ST == ST_FP8)
                    __builtin_nontemporal_store(code[nt][0], reinterpret_cast<uint32_t *>(cp + byte));
                else
                    *reinterpret_cast<uint16_t *>(cp + byte) = (uint16_t)code[nt][0];
            }
        }
    }

    // Last wavefront of its group: the group arrives at the sequence's
    // counter; the last group means every wavefront of the sequence has read base.
    if (lane == 0 && prev == r.H / r.G / HC * NW - 1) {
        int32_t *seq = args.sync + (size_t)b * (r.G + 1) * kSyncStride;
        atomicExch(seq + (size_t)g * kSyncStride, 0);
        if (atomicAdd(seq + (size_t)r.G * kSyncStride, 1) == r.G - 1) {
            atomicExch(seq + (size_t)r.G * kSyncStride, 0);
            args.base_out[b] = pos;
        }
    }
}

template <int P, int N, int ST, int LM, int HC>
static hipError_t launch_shared_hc(const FlushArgs &a, hipStream_t s) {
    const unsigned blocks = (unsigned)((size_t)a.r.B * a.r.H / HC);
    if (a.r.io_bf16)
        flush_shared_kernel<P, N, ST, true, LM, HC><<<blocks, P / 16 * 64, 0, s>>>(a);
    else
        flush_shared_kernel<P, N, ST, false, LM, HC><<<blocks, P / 16 * 64, 0, s>>>(a);
    return hipGetLastError();
}

// Two heads per workgroup, every load issued up front, for flushes that
// fold full rings only (as for the vector fold); one otherwise.  Four heads
// measured the same for e4m3 and FP4 and slower for bf16 (registers).
template <int P, int N, int ST, int LM>
static hipError_t launch_shared_lm(const FlushArgs &a, hipStream_t s) {
    constexpr int HC = P < 64 ? 1 : 2;
    if (HC > 1 && a.min_count >= a.r.L && (a.r.H / a.r.G) % HC == 0) return launch_shared_hc<P, N, ST, LM, HC>(a, s);
    return launch_shared_hc<P, N, ST, LM, 1>(a, s);
}

template <int P, int N, int ST>
static hipError_t launch_shared(const FlushArgs &a, hipStream_t s) {
    return a.r.L <= 16 ? launch_shared_lm<P, N, ST, 16>(a, s) : launch_shared_lm<P, N, ST, kMaxRing>(a, s);
}

hipError_t launch_flush_shared(int P, int N, int st, const FlushArgs &a, hipStream_t s) {
    if (a.force_empty || a.S_out) return hipErrorInvalidValue;   // a fold of the copy, in place
    auto pn = [&](auto launch3) -> hipError_t {
        switch (st) {
            case ST_BF16: return launch3(std::integral_constant<int, ST_BF16>{});
            case ST_FP8: return launch3(std::integral_constant<int, ST_FP8>{});
            case ST_FP4: return launch3(std::integral_constant<int, ST_FP4>{});
            default: return hipErrorInvalidValue;
        }
    };
    if (P == 16 && N == 16) return pn([&](auto t) { return launch_shared<16, 16, decltype(t)::value>(a, s); });
    if (P == 64 && N == 64) return pn([&](auto t) { return launch_shared<64, 64, decltype(t)::value>(a, s); });
    if (P == 64 && N == 128) return pn([&](auto t) { return launch_shared<64, 128, decltype(t)::value>(a, s); });
    if (P == 128 && N == 128) return pn([&](auto t) { return launch_shared<128, 128, decltype(t)::value>(a, s); });
    return hipErrorInvalidValue;
}

}  // namespace replay
