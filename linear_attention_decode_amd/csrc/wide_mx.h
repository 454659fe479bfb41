// wide_mx.h -- S Q^T for a window of up to 16 queries on the matrix cores
// (queries in LDS as bf16 for bf16 io; float32 io takes dot_f32q),
// shared by the matrix-core verify kernel (verify_wide.hip) and the fused
// verify round (verify_step.hip), so that both produce the same bits:
//   - streaming wavefront i owns rows 16i..16i+15 of a head's tile;
//   - coalesced staging (16-byte lane steps, rows of whole 128-byte lines):
//     the rows are read in 128-byte segments, 8 lanes to a cache line, and
//     each 16-row x 128-byte chunk is turned into the operand layout through
//     the wavefront's own LDS buffer.  Loading the operand layout directly
//     makes every load instruction touch 16 half lines, twice the cache
//     requests; other shapes (rows shorter than a line) do load it directly;
//   - operand layout: lane (row r = lane % 16, group g = lane / 16) holds,
//     at step st, 16 bytes of row 16i + r starting at column (4 st + g) CVEC
//     (the contraction order is free, so a lane's 16 bytes are contiguous);
//   - D = S Q^T for the 16 rows, Q[w][n] in LDS as bf16 (rows past the
//     window zero):
//       float32 tiles: v_mfma_f32_16x16x4_f32, four per 16 columns: the t-th
//         takes column (4 st + g) 4 + t in lane group g;
//       bf16 tiles: v_mfma_f32_16x16x32_bf16, columns (4 st + g) 8 .. +7;
//       e4m3 tiles: 16 codes a lane cover two such products, turned into
//         bf16 pairs by the hardware conversion (exact);
//       MX FP4 tiles: step st is MX block st of the row (32 codes, 8 a lane
//         group, 4 bytes a lane), one product per block into an accumulator
//         of its own, scaled by the block's 2^e afterwards (exact) and added
//         block after block: no per-row scale ever meets another row's;
//       N below 32: the bf16, e4m3 and FP4 values are widened (FP4 with its
//         block's scale, exact) and take the float32 products;
//   - D[p][w] sits in lane (4-row group, column w), register rr -> row
//     16i + 4g + rr.
#pragma once
#include <type_traits>

#include "ring_mx.h"

namespace replay {

constexpr int kWide = 16;   // columns of D (queries), the MFMA tile width

template <int ST, int N>
constexpr bool wide_bf16_path() { return ST != ST_F32 && N % 32 == 0; }

template <int P, int N, int ST>
struct WideTile {
    static constexpr bool BF = wide_bf16_path<ST, N>();
    static constexpr int NTS = (P / 16) * 64;                      // one wavefront per 16 rows
    static constexpr bool MX = ST == ST_FP4;
    static constexpr int ESZ = ST == ST_F32 ? 4 : (ST == ST_BF16 ? 2 : 1);   // FP4: two codes a byte
    static constexpr int CVEC = BF ? (MX ? 8 : 16 / ESZ) : 4;      // elements a lane loads per step
    static constexpr int STEPS = N / (4 * CVEC);                   // loads per lane (4 lane groups)
    static constexpr int NB = N / 32;                              // MX blocks of a row (FP4)
    static constexpr int TS = N + 8;                               // LDS row stride of Q (bf16), in elements
    static constexpr int RB = MX ? N / 2 : N * ESZ;                // bytes of a tile row
    static constexpr bool COAL = !MX && (ST == ST_F32 || BF) && RB % 128 == 0;
    static constexpr int TROW = 36;   // staging row stride in words (128 bytes + 16 of padding: the
                                      // column reads of 16 rows hit distinct banks)
    using TE = uint16_t;   // Q stays bf16 in LDS (widened exactly where the float32 products take it)
    static_assert(!COAL || STEPS == 2 * (RB / 128), "two load steps per 128-byte chunk");
    static_assert(P % 16 == 0 && N % 16 == 0 && N % (4 * CVEC) == 0, "tile shape");
};

// A lane's share of one load step of the tile: CVEC elements of one row.
template <int ST, bool BF>
struct WideA;

template <>
struct WideA<ST_F32, false> {   // 4 floats
    f32x4 v;
    __device__ __forceinline__ void load(const void *S, size_t e) {
        v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(static_cast<const float *>(S) + e));
    }
    __device__ __forceinline__ void set(uint4 u) { v = __builtin_bit_cast(f32x4, u); }
    __device__ __forceinline__ f32x4 f32() const { return v; }
};
template <>
struct WideA<ST_BF16, false> {   // 4 bf16, widened
    u32x2 v;
    __device__ __forceinline__ void load(const void *S, size_t e) {
        v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(S) + e));
    }
    __device__ __forceinline__ f32x4 f32() const {
        return f32x4{bf16_bits_to_f32(v.x & 0xffffu), bf16_bits_to_f32(v.x >> 16), bf16_bits_to_f32(v.y & 0xffffu),
                     bf16_bits_to_f32(v.y >> 16)};
    }
};
template <>
struct WideA<ST_FP8, false> {   // 4 e4m3 codes, widened (unscaled)
    uint32_t v;
    __device__ __forceinline__ void load(const void *S, size_t e) {
        v = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(static_cast<const uint8_t *>(S) + e));
    }
    __device__ __forceinline__ f32x4 f32() const {
        float x[4];
        fp8x4_to_f32(v, x);
        return f32x4{x[0], x[1], x[2], x[3]};
    }
};
template <>
struct WideA<ST_FP4, false> {   // 4 E2M1 codes of one MX block, widened with the block's scale (exact)
    uint32_t v;
    int se;
    __device__ __forceinline__ void load_mx(const void *S, const void *scales, size_t e) {
        v = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(static_cast<const uint8_t *>(S) + e / 2));
        se = (int)static_cast<const uint8_t *>(scales)[e / 32] - 127;
    }
    __device__ __forceinline__ f32x4 f32() const {
        float x[4];
        fp4_pair_to_f32(v, 0, x);
        fp4_pair_to_f32(v, 1, x + 2);
        return f32x4{ldexpf(x[0], se), ldexpf(x[1], se), ldexpf(x[2], se), ldexpf(x[3], se)};
    }
};
template <>
struct WideA<ST_FP4, true> {   // 8 E2M1 codes (4 bytes) of one MX block, unscaled
    uint32_t v;
    __device__ __forceinline__ void load(const void *S, size_t e) {
        v = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(static_cast<const uint8_t *>(S) + e / 2));
    }
    // the 8 codes as bf16 pairs (exact)
    __device__ __forceinline__ uint4 bf16x8() const {
        return uint4{fp4_pair_to_bf16(v, 0), fp4_pair_to_bf16(v, 1), fp4_pair_to_bf16(v, 2), fp4_pair_to_bf16(v, 3)};
    }
    // the 8 codes' values (unscaled, exact)
    __device__ __forceinline__ void widen(float *x) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) fp4_pair_to_f32(v, i, x + 2 * i);
    }
};
template <int ST>
struct WideA<ST, true> {   // 16 bytes: 8 bf16, or 16 e4m3 codes
    uint4 v;
    __device__ __forceinline__ void load(const void *S, size_t e) {
        const char *p = static_cast<const char *>(S) + e * (ST == ST_BF16 ? 2 : 1);
        const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
        v = uint4{w.x, w.y, w.z, w.w};
    }
    __device__ __forceinline__ void set(uint4 u) { v = u; }
    // the values (e4m3: unscaled), widened exactly: 8 (bf16) or 16 (e4m3)
    __device__ __forceinline__ void widen(float *x) const {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (ST == ST_BF16) {
                x[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
                x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
            } else {
                fp8x4_to_f32(w[i], x + 4 * i);
            }
        }
    }
    // e4m3: codes 8h..8h+7 as bf16 pairs (exact)
    __device__ __forceinline__ uint4 bf16_half(int h) const {
        const uint32_t w0 = h ? v.z : v.x, w1 = h ? v.w : v.y;
        return uint4{bf16_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false)),
                     bf16_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true)),
                     bf16_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false)),
                     bf16_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true))};
    }
};

// One lane's part of a streaming wavefront's 16 rows.
template <int P, int N, int ST>
struct WideRows {
    using WT = WideTile<P, N, ST>;
    static constexpr int STEPS = WT::STEPS;
    WideA<ST, WT::BF> at[STEPS];        // operand layout
    uint4 raw[WT::COAL ? STEPS : 1];    // coalesced: load i = rows 8 (i & 1) + lane / 8,
                                        // bytes 128 (i >> 1) + 16 (lane % 8)

    // Issue every load of rows p0..p0+15 of the tile that starts at element
    // `tile` of S (`scales`: the E8M0 block scales of an FP4 copy).
    __device__ __forceinline__ void load(const void *S, size_t tile, int p0, int lane, const void *scales = nullptr) {
        if constexpr (WT::COAL) {
            const char *t = static_cast<const char *>(S) + (tile + (size_t)p0 * N) * WT::ESZ;
#pragma unroll
            for (int i = 0; i < STEPS; ++i) {
                const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                    t + (size_t)(8 * (i & 1) + (lane >> 3)) * WT::RB + 128 * (i >> 1) + 16 * (lane & 7)));
                raw[i] = uint4{w.x, w.y, w.z, w.w};
            }
        } else {
            const size_t row = tile + (size_t)(p0 + (lane & 15)) * N;
#pragma unroll
            for (int st = 0; st < STEPS; ++st) {
                const size_t e = row + (size_t)(4 * st + (lane >> 4)) * WT::CVEC;
                if constexpr (ST == ST_FP4 && !WT::BF)
                    at[st].load_mx(S, scales, e);
                else
                    at[st].load(S, e);
            }
        }
    }

    // float32 tiles: f(x, r, c) on each of this lane's 4-float vectors, x the
    // values of row p0 + r, columns c..c+3 (in whichever layout holds them)
    template <class F>
    __device__ __forceinline__ void each_f32(int lane, F f) {
        static_assert(ST == ST_F32, "float32 tiles");
        if constexpr (WT::COAL) {
#pragma unroll
            for (int i = 0; i < STEPS; ++i) {
                f32x4 x = __builtin_bit_cast(f32x4, raw[i]);
                f(x, 8 * (i & 1) + (lane >> 3), 32 * (i >> 1) + 4 * (lane & 7));
                raw[i] = __builtin_bit_cast(uint4, x);
            }
        } else {
#pragma unroll
            for (int st = 0; st < STEPS; ++st) f(at[st].v, lane & 15, 4 * (4 * st + (lane >> 4)));
        }
    }

    // coalesced: into the operand layout, chunk by chunk through this
    // wavefront's buffer T (lane (row lr, group lg) of step st reads row lr,
    // bytes 64 (st % 2) + 16 lg of chunk st / 2; wave_lds_sync puts every
    // lane's writes of a chunk before any lane's reads, and those reads
    // before the next chunk's writes)
    __device__ __forceinline__ void transpose(uint32_t (*T)[WT::TROW], int lane) {
        if constexpr (WT::COAL) {
            const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
            for (int c = 0; c < STEPS / 2; ++c) {
                if (c > 0) wave_lds_sync();
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
                    *reinterpret_cast<uint4 *>(&T[8 * hf + (lane >> 3)][4 * (lane & 7)]) = raw[2 * c + hf];
                wave_lds_sync();
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                    at[2 * c + s2].set(*reinterpret_cast<const uint4 *>(&T[lr][16 * s2 + 4 * lg]));
            }
        }
    }

    // MX FP4 (N a multiple of 32): D = S Q^T over the 16 rows, one product
    // per block, each scaled by its 2^e; rsc = the block scales of row
    // p0 + 4 lg (4 rows of NB bytes, this lane's output rows).
    __device__ __forceinline__ f32x4 dot_mx(const typename WT::TE (*s_Q)[WT::TS], int lane,
                                            const uint8_t *rsc) const {
        static_assert(ST == ST_FP4 && WT::BF && (WT::NB == 2 || WT::NB == 4), "MX blocks");
        const int lr = lane & 15, lg = lane >> 4;
        uint32_t sw[WT::NB];   // the 4 rows' scale bytes, rsc[rr * NB + st]
        if constexpr (WT::NB == 4) {
            const uint4 u = *reinterpret_cast<const uint4 *>(rsc);
            sw[0] = u.x; sw[1] = u.y; sw[2] = u.z; sw[3] = u.w;
        } else {
            const uint2 u = *reinterpret_cast<const uint2 *>(rsc);
            sw[0] = u.x; sw[1] = u.y;
        }
        auto se = [&](int rr, int st) {   // scale byte rr * NB + st
            const int i = rr * WT::NB + st;
            return (int)((sw[i >> 2] >> (8 * (i & 3))) & 0xffu) - 127;
        };
        f32x4 out = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const uint4 q = *reinterpret_cast<const uint4 *>(&s_Q[lr][(4 * st + lg) * WT::CVEC]);
            const f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(at[st].bf16x8()), as_bf16x8(q),
                                                                      f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) out[rr] += ldexpf(acc[rr], se(rr, st));
        }
        return out;
    }

    // float32 queries (float32 io): D = S Q^T over the 16 rows with
    // v_mfma_f32_16x16x4_f32, every tile value widened exactly; product t of
    // step st takes column c0 + t of the lane's CVEC columns c0 = (4 st + lg)
    // CVEC.  MX FP4 with whole blocks per row: one accumulator per block,
    // scaled by the block's 2^e (rsc as for dot_mx).  Register rr = D[4 lg + rr][lr].
    template <int TSF>
    __device__ __forceinline__ f32x4 dot_f32q(const float (*s_Qf)[TSF], int lane, const uint8_t *rsc) const {
        constexpr bool MXB = ST == ST_FP4 && WT::BF;
        constexpr int CV = WT::CVEC;
        const int lr = lane & 15, lg = lane >> 4;
        uint32_t sw[MXB ? WT::NB : 1];
        if constexpr (MXB) {
            static_assert(WT::NB == 2 || WT::NB == 4, "MX blocks");
            if constexpr (WT::NB == 4) {
                const uint4 u = *reinterpret_cast<const uint4 *>(rsc);
                sw[0] = u.x; sw[1] = u.y; sw[2] = u.z; sw[3] = u.w;
            } else {
                const uint2 u = *reinterpret_cast<const uint2 *>(rsc);
                sw[0] = u.x; sw[1] = u.y;
            }
        }
        f32x4 out = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const int c0 = (4 * st + lg) * CV;
            float x[CV];
            if constexpr (!WT::BF) {
                const f32x4 a = at[st].f32();
                x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
            } else {
                at[st].widen(x);
            }
            f32x4 acc = MXB ? f32x4{0.f, 0.f, 0.f, 0.f} : out;
#pragma unroll
            for (int t4 = 0; t4 < CV / 4; ++t4) {
                const f32x4 q = *reinterpret_cast<const f32x4 *>(&s_Qf[lr][c0 + 4 * t4]);
#pragma unroll
                for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[4 * t4 + u], q[u], acc, 0, 0, 0);
            }
            if constexpr (MXB) {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int i = rr * WT::NB + st;
                    out[rr] += ldexpf(acc[rr], (int)((sw[i >> 2] >> (8 * (i & 3))) & 0xffu) - 127);
                }
            } else {
                out = acc;
            }
        }
        return out;
    }

    // D = S Q^T over the 16 rows: register rr = D[4 lg + rr][lr]
    __device__ __forceinline__ f32x4 dot(const typename WT::TE (*s_Q)[WT::TS], int lane) const {
        static_assert(!(ST == ST_FP4 && WT::BF), "FP4 tiles with whole blocks per row take dot_mx");
        const int lr = lane & 15, lg = lane >> 4;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const int c0 = (4 * st + lg) * WT::CVEC;   // first column of this lane's step
            if constexpr (!WT::BF) {
                const f32x4 a = at[st].f32();
                const u32x2 qq = *reinterpret_cast<const u32x2 *>(&s_Q[lr][c0]);
                const f32x4 q = {bf16_bits_to_f32(qq.x & 0xffffu), bf16_bits_to_f32(qq.x >> 16),
                                 bf16_bits_to_f32(qq.y & 0xffffu), bf16_bits_to_f32(qq.y >> 16)};
#pragma unroll
                for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], q[t], acc, 0, 0, 0);
            } else if constexpr (ST == ST_BF16) {
                const uint4 q = *reinterpret_cast<const uint4 *>(&s_Q[lr][c0]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(at[st].v), as_bf16x8(q), acc, 0, 0, 0);
            } else {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const uint4 q = *reinterpret_cast<const uint4 *>(&s_Q[lr][c0 + 8 * hh]);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(at[st].bf16_half(hh)), as_bf16x8(q), acc,
                                                                  0, 0, 0);
                }
            }
        }
        return acc;
    }
};

// Columns n..n+7 of row w of Q: 8 bf16 (one 16-byte word).
template <int P, int N, int ST, class QRows>
__device__ __forceinline__ void wide_put_q(QRows s_Q, int w, int n, uint4 u) {
    *reinterpret_cast<uint4 *>(&s_Q[w][n]) = u;
}

// One output: abar_w (sc (S q_w)[p]) + R[w][p] (sc: the e4m3 scale, else 1).
__device__ __forceinline__ float wide_out(float ab, float sc, float acc, float rt) { return ab * (sc * acc) + rt; }

}  // namespace replay
