// device_common.h -- device helpers for the gfx950 kernels of libreplayssm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace replay {

// ---- workgroup -> work mapping ------------------------------------------
// The dispatcher hands workgroup i to XCD (i mod 8).  Remapping gives each
// XCD a contiguous range of logical ids, so heads that share a group's k/q
// ring (consecutive ids) run on the same XCD and share its L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    constexpr int kXcd = 8;
    const int x = bid % kXcd, local = bid / kXcd;
    const int q = nblocks / kXcd, r = nblocks % kXcd;
    return x * q + (x < r ? x : r) + local;
}

// ---- number formats ------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

// float32 -> bf16 bits, round to nearest even, NaN kept quiet (a select,
// not a branch: the conversion sits in unrolled per-element loops).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    return (u & 0x7fffffffu) > 0x7f800000u ? (u >> 16) | 0x40u : rounded;
}

// two floats -> a bf16 pair (a in the low half), round to nearest even, by
// the hardware conversion (v_cvt_pk_bf16_f32)
typedef __bf16 bf16x2_pair_t __attribute__((ext_vector_type(2)));
typedef float f32x2_pair_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16_pair(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_pair_t{a, b}, bf16x2_pair_t));
}

// four e4m3 codes packed in a word -> floats (hardware OCP e4m3 conversion)
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float *out) {
    auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    out[0] = lo[0];
    out[1] = lo[1];
    out[2] = hi[0];
    out[3] = hi[1];
}

// x / d for many x and one divisor d, for e4m3 codes.  The correctly rounded
// float32 division runs a reciprocal refined by one Newton step, two
// remainder corrections and a special-case fix-up, after rescaling operands
// whose exponents are near the ends of the range; here the divisor's part is
// formed once.  While 2^-60 <= d <= 2^60 and |x| <= 448 d, that rescaling
// only ever applies to quotients below 2^-43 (|x| < 2^-103, or x / d
// subnormal), so the result has the bits of x / d wherever they can decide an
// e4m3 code (those small quotients are +-0 in e4m3 either way, sign from
// the fix-up).  Outside that range of d, exact division.  d must be the
// same in every lane; run(f) calls f with the division to use, so that the
// choice is one scalar branch around the caller's whole loop.
struct ScaleDiv {
    float d, y;
    __device__ __forceinline__ explicit ScaleDiv(float d_) : d(d_) {
        const float y0 = __builtin_amdgcn_rcpf(d);
        y = fmaf(fmaf(-d, y0, 1.0f), y0, y0);
    }
    __device__ __forceinline__ float quick(float x) const {
        float q = x * y;
        q = fmaf(fmaf(-d, q, x), y, q);
        q = fmaf(fmaf(-d, q, x), y, q);
        return __builtin_amdgcn_div_fixupf(q, d, x);
    }
    template <class F>
    __device__ __forceinline__ void run(F f) const {
        const int fast = __builtin_amdgcn_readfirstlane((int)(d >= 0x1p-60f && d <= 0x1p60f));
        if (fast)
            f([this](float x) { return quick(x); });
        else
            f([this](float x) { return x / d; });
    }
};

// four floats -> packed e4m3 codes, round to nearest even, saturating to +-448
__device__ __forceinline__ uint32_t f32x4_to_fp8(float a, float b, float c, float d) {
    a = __builtin_amdgcn_fmed3f(a, 448.0f, -448.0f);
    b = __builtin_amdgcn_fmed3f(b, 448.0f, -448.0f);
    c = __builtin_amdgcn_fmed3f(c, 448.0f, -448.0f);
    d = __builtin_amdgcn_fmed3f(d, 448.0f, -448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// MX FP4 block of 32 values whose largest magnitude is amax: the E8M0
// exponent se of its scale X = 2^se = 2^(floor(log2 amax) - 2), clamped to
// the format's range; -127 for an all-zero block.
__device__ __forceinline__ int mxfp4_block_exp(float amax) {
    if (!(amax > 0.f)) return -127;
    int ex;
    (void)frexpf(amax, &ex);   // amax = f 2^ex, f in [0.5, 1)
    return ex - 3 < -127 ? -127 : (ex - 3 > 127 ? 127 : ex - 3);
}

// Four values of a block with exponent se -> two bytes of E2M1 codes of
// value / 2^se (the division exact by ldexp; the hardware conversion rounds
// to nearest even and saturates at 6), first value in the low nibble.
__device__ __forceinline__ uint16_t mxfp4_codes4(float a, float b, float c, float d, int se) {
    const uint32_t lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, ldexpf(a, -se), ldexpf(b, -se), 1.0f, 0);
    const uint32_t hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, ldexpf(c, -se), ldexpf(d, -se), 1.0f, 0);
    return (uint16_t)((lo & 0xffu) | ((hi & 0xffu) << 8));
}

// ---- io loads (q, k, v: float32 or bf16, fixed at compile time) ----------
// Load 4 consecutive io elements starting at element index `i` (i % 4 == 0).
template <bool BF16>
__device__ __forceinline__ void load_io4(const void *base, size_t i, float *out) {
    if constexpr (BF16) {
        const uint2 w = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(base) + i);
        out[0] = bf16_bits_to_f32(w.x & 0xffffu);
        out[1] = bf16_bits_to_f32(w.x >> 16);
        out[2] = bf16_bits_to_f32(w.y & 0xffffu);
        out[3] = bf16_bits_to_f32(w.y >> 16);
    } else {
        const float4 f = *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + i);
        out[0] = f.x;
        out[1] = f.y;
        out[2] = f.z;
        out[3] = f.w;
    }
}

// Load 8 consecutive io elements starting at element index `i` (i % 8 == 0).
template <bool BF16>
__device__ __forceinline__ void load_io8(const void *base, size_t i, float *out) {
    if constexpr (BF16) {
        const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + i);
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            out[2 * k] = bf16_bits_to_f32(u[k] & 0xffffu);
            out[2 * k + 1] = bf16_bits_to_f32(u[k] >> 16);
        }
    } else {
        load_io4<false>(base, i, out);
        load_io4<false>(base, i + 4, out + 4);
    }
}

template <bool BF16>
__device__ __forceinline__ float load_io1(const void *base, size_t i) {
    if constexpr (BF16) return bf16_bits_to_f32(static_cast<const uint16_t *>(base)[i]);
    return static_cast<const float *>(base)[i];
}

// Raw io vectors: E consecutive io elements loaded as raw bits and widened
// to float only where they are used, so a load never forces a wait at the
// place it is issued.
template <bool BF16, int E>
struct IoVec;

template <>
struct IoVec<true, 8> {
    uint4 r;
    __device__ __forceinline__ void load(const void *base, size_t i) {
        r = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + i);
    }
    __device__ __forceinline__ void widen(float *out) const {
        const uint32_t u[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            out[2 * k] = bf16_bits_to_f32(u[k] & 0xffffu);
            out[2 * k + 1] = bf16_bits_to_f32(u[k] >> 16);
        }
    }
};

template <>
struct IoVec<false, 8> {
    float4 a, b;
    __device__ __forceinline__ void load(const void *base, size_t i) {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(base) + i);
        a = p[0];
        b = p[1];
    }
    __device__ __forceinline__ void widen(float *out) const {
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
        out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    }
};

template <>
struct IoVec<true, 4> {
    uint2 r;
    __device__ __forceinline__ void load(const void *base, size_t i) {
        r = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(base) + i);
    }
    __device__ __forceinline__ void widen(float *out) const {
        out[0] = bf16_bits_to_f32(r.x & 0xffffu);
        out[1] = bf16_bits_to_f32(r.x >> 16);
        out[2] = bf16_bits_to_f32(r.y & 0xffffu);
        out[3] = bf16_bits_to_f32(r.y >> 16);
    }
};

template <>
struct IoVec<false, 4> {
    float4 a;
    __device__ __forceinline__ void load(const void *base, size_t i) {
        a = *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + i);
    }
    __device__ __forceinline__ void widen(float *out) const {
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    }
};

// Buffer resource over [base, base + bytes) (bytes < 2^32).  A load through
// it takes a 32-bit per-lane byte offset and a wave-uniform byte offset held
// in a scalar register, so a wavefront that reads many rows of one region
// keeps a single address register instead of a 64-bit address per load.
// Offsets at or past `bytes` read zero.  Word 3 is the gfx9-family setting
// for untyped (raw) buffer access.  `base` and `bytes` must be the same in
// every lane: they are taken from the first active lane, so the descriptor
// is built in scalar registers even where the compiler cannot prove the
// address uniform (it would otherwise wrap each load in a loop over the
// lanes' distinct descriptors).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void *ub = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

template <>
struct IoVec<true, 1> {
    uint32_t r;
    __device__ __forceinline__ void load(const void *base, size_t i) { r = static_cast<const uint16_t *>(base)[i]; }
    __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
        r = __builtin_amdgcn_raw_buffer_load_b16(rs, voff, soff, 0);
    }
    __device__ __forceinline__ float value() const { return bf16_bits_to_f32(r); }
};

template <>
struct IoVec<false, 1> {
    float r;
    __device__ __forceinline__ void load(const void *base, size_t i) { r = static_cast<const float *>(base)[i]; }
    __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
        r = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0));
    }
    __device__ __forceinline__ float value() const { return r; }
};

// k . q over 8 io elements held raw.  bf16 pairs go through the packed bf16
// dot instruction (v_dot2c_f32_bf16: the products of bf16 values are exact in
// float32), float32 elements through an FMA chain; no widened copies are
// kept in registers.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot8(const IoVec<true, 8> &k, const IoVec<true, 8> &q) {
    float d = 0.f;
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.r.x), __builtin_bit_cast(bf16x2_t, q.r.x), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.r.y), __builtin_bit_cast(bf16x2_t, q.r.y), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.r.z), __builtin_bit_cast(bf16x2_t, q.r.z), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.r.w), __builtin_bit_cast(bf16x2_t, q.r.w), d, false);
    return d;
}

__device__ __forceinline__ float dot8(const IoVec<false, 8> &k, const IoVec<false, 8> &q) {
    float d = 0.f;
    d = fmaf(k.a.x, q.a.x, d);
    d = fmaf(k.a.y, q.a.y, d);
    d = fmaf(k.a.z, q.a.z, d);
    d = fmaf(k.a.w, q.a.w, d);
    d = fmaf(k.b.x, q.b.x, d);
    d = fmaf(k.b.y, q.b.y, d);
    d = fmaf(k.b.z, q.b.z, d);
    d = fmaf(k.b.w, q.b.w, d);
    return d;
}

// Ring slot of entry j (0-based, oldest first) for a ring that starts at
// slot bmod = base mod L; valid for 0 <= j < L.
__device__ __forceinline__ int ring_slot(int bmod, int j, int L) {
    const int s = bmod + j;
    return s >= L ? s - L : s;
}

// Native vector types (the nontemporal builtins take these, not HIP's
// struct vectors).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// a*b over a bf16 pair each (raw bits, element 0 in the low half) plus acc,
// by the packed bf16 dot instruction (the products are exact in float32)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), acc,
                                          false);
}

template <typename V>
__device__ __forceinline__ uint32_t bf16_pair_bits(V v) { return __builtin_bit_cast(uint32_t, v); }

// ---- state tile chunks ---------------------------------------------------
// A chunk is VEC consecutive elements of one state row, loaded with one
// vector load and widened to float.
template <int ST, int VEC>
struct Chunk;

template <int VEC>
struct Chunk<ST_F32, VEC> {
    static_assert(VEC == 4, "f32 chunks are 16 bytes");
    f32x4 raw;
    __device__ __forceinline__ void load(const void *S, size_t e) {
        raw = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(static_cast<const float *>(S) + e));
    }
    __device__ __forceinline__ void widen(float *out, float) const {
        out[0] = raw.x; out[1] = raw.y; out[2] = raw.z; out[3] = raw.w;
    }
};

template <int VEC>
struct Chunk<ST_BF16, VEC> {
    static_assert(VEC == 8 || VEC == 4, "bf16 chunks are 16 or 8 bytes");
    uint32_t raw[VEC / 2];
    __device__ __forceinline__ void load(const void *S, size_t e) {
        const uint16_t *p = static_cast<const uint16_t *>(S) + e;
        if constexpr (VEC == 8) {
            u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
            raw[0] = w.x; raw[1] = w.y; raw[2] = w.z; raw[3] = w.w;
        } else {
            u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
            raw[0] = w.x; raw[1] = w.y;
        }
    }
    __device__ __forceinline__ void widen(float *out, float) const {
#pragma unroll
        for (int i = 0; i < VEC / 2; ++i) {
            out[2 * i] = bf16_bits_to_f32(raw[i] & 0xffffu);
            out[2 * i + 1] = bf16_bits_to_f32(raw[i] >> 16);
        }
    }
    // sum_e x[e] q[e] with q given as VEC/2 words of bf16 pairs (element order)
    __device__ __forceinline__ float dot_bf16(const uint32_t *q) const {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < VEC / 2; ++i) acc = dot2_bf16(raw[i], q[i], acc);
        return acc;
    }
};

template <int VEC>
struct Chunk<ST_FP8, VEC> {
    static_assert(VEC == 16 || VEC == 8 || VEC == 4, "e4m3 chunks are 16, 8 or 4 bytes");
    uint32_t raw[VEC / 4];
    __device__ __forceinline__ void load(const void *S, size_t e) {
        const uint8_t *p = static_cast<const uint8_t *>(S) + e;
        if constexpr (VEC == 16) {
            u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
            raw[0] = w.x; raw[1] = w.y; raw[2] = w.z; raw[3] = w.w;
        } else if constexpr (VEC == 8) {
            u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
            raw[0] = w.x; raw[1] = w.y;
        } else {
            raw[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
        }
    }
    // widened values are the codes' values times the per-head scale
    __device__ __forceinline__ void widen(float *out, float scale) const {
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i) {
            fp8x4_to_f32(raw[i], out + 4 * i);
        }
#pragma unroll
        for (int i = 0; i < VEC; ++i) out[i] *= scale;
    }
    // sum_e code[e] q[e] (unscaled), q as VEC/2 words of bf16 pairs: each code
    // pair goes to a bf16 pair (exact: e4m3 values are bf16 values)
    __device__ __forceinline__ float dot_bf16(const uint32_t *q) const {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i) {
            acc = dot2_bf16(bf16_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[i], 1.0f, false)),
                            q[2 * i], acc);
            acc = dot2_bf16(bf16_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[i], 1.0f, true)),
                            q[2 * i + 1], acc);
        }
        return acc;
    }
};

// Two E2M1 codes (byte `sel` of w) -> their float values (hardware conversion, scale 1).
__device__ __forceinline__ void fp4_pair_to_f32(uint32_t w, int sel, float *out) {
    decltype(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0)) v;
    switch (sel) {
        case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); break;
        case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); break;
        case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); break;
        default: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); break;
    }
    out[0] = v[0];
    out[1] = v[1];
}

// Two E2M1 codes (byte `sel` of w) -> a bf16 pair (exact), as raw bits.
__device__ __forceinline__ uint32_t fp4_pair_to_bf16(uint32_t w, int sel) {
    switch (sel) {
        case 0: return bf16_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
        case 1: return bf16_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
        case 2: return bf16_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
        default: return bf16_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
    }
}

// MX FP4 chunk: VEC codes (VEC/2 bytes) of one block of 32 values, with the
// block's E8M0 scale exponent.  widen() gives the unscaled E2M1 values (the
// hardware conversion, exact); callers multiply sums by 2^se, which is exact
// for a power of two, so a block's products are formed once and scaled once.
template <int VEC>
struct Chunk<ST_FP4, VEC> {
    static_assert(VEC == 32 || VEC == 16 || VEC == 8 || VEC == 4, "FP4 chunks are 16, 8, 4 or 2 bytes");
    static constexpr int WORDS = VEC >= 8 ? VEC / 8 : 1;
    uint32_t raw[WORDS];
    int se;
    // e: element index of the chunk's first value; scales: one byte per block of 32
    __device__ __forceinline__ void load_mx(const void *S, const void *scales, size_t e) {
        load_codes(S, e);
        se = (int)static_cast<const uint8_t *>(scales)[e / 32] - 127;
    }
    // the codes alone (the caller sets se)
    __device__ __forceinline__ void load_codes(const void *S, size_t e) {
        const uint8_t *p = static_cast<const uint8_t *>(S) + e / 2;
        if constexpr (VEC == 32) {
            u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
            raw[0] = w.x; raw[1] = w.y; raw[2] = w.z; raw[3] = w.w;
        } else if constexpr (VEC == 16) {
            u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
            raw[0] = w.x; raw[1] = w.y;
        } else if constexpr (VEC == 8) {
            raw[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
        } else {
            raw[0] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(p));
        }
    }
    __device__ __forceinline__ void widen(float *out, float) const {
#pragma unroll
        for (int i = 0; i < VEC / 2; ++i) fp4_pair_to_f32(raw[i / 4], i % 4, out + 2 * i);
    }
    // sum_e code[e] q[e] (unscaled), q as VEC/2 words of bf16 pairs
    __device__ __forceinline__ float dot_bf16(const uint32_t *q) const {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < VEC / 2; ++i) acc = dot2_bf16(fp4_pair_to_bf16(raw[i / 4], i % 4), q[i], acc);
        return acc;
    }
};

// ---- lane exchanges --------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Value of the partner lane for a butterfly step on lane bit `bit`.  The
// partner differs from this lane in `bit` and possibly in lower bits, never
// in higher ones: bit 0 -> lane^1, bit 1 -> lane^2 (quad permutes), bit 2 ->
// lane^7 (row half-mirror), bit 3 -> lane^15 (row mirror), bits 4, 5 ->
// lane^16, lane^32 (ds_bpermute).  Reduction steps taken from the top bit
// down therefore always combine lanes that hold the same partial set, and a
// full sequence of steps covers every lane of the group.
__device__ __forceinline__ float lane_partner(float x, int bit) {
    switch (bit) {
        case 0: return dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
        case 1: return dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
        case 2: return dpp_mov<0x141>(x);   // row_half_mirror
        case 3: return dpp_mov<0x140>(x);   // row_mirror
        case 4: return __shfl_xor(x, 16);
        default: return __shfl_xor(x, 32);
    }
}

// Value of lane `lane` (a wavefront-uniform index) broadcast to all lanes.
__device__ __forceinline__ float bcast(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Sum over aligned groups of TS lanes (TS a power of two, <= 64); every lane
// of the group gets the sum.
template <int TS>
__device__ __forceinline__ float group_sum(float x) {
    constexpr int K = __builtin_ctz(TS);
#pragma unroll
    for (int bit = K - 1; bit >= 0; --bit) x += lane_partner(x, bit);
    return x;
}

// ---- reductions over the lanes that share a state row --------------------
// v[i][w] holds a lane's partial sum for row-slot i (ITER of them) and query
// w.  The LPR lanes of a row group (aligned, inside one wavefront) cover one
// row each iteration.  Halving steps exchange half of the remaining row-slots
// with the partner lane (top lane bits first), so every exchange moves useful
// data; once a single slot is left, plain butterfly steps finish it.  On
// return slots 0..FINAL-1 are complete; slot e of a lane stands for original
// row-slot  e + FINAL * halving_index(lane).
template <int ITER, int LPR>
struct RowReduce {
    static constexpr int K = __builtin_ctz(LPR);            // lane bits of a group
    static constexpr int I = __builtin_ctz(ITER);
    static constexpr int NH = (I < K) ? I : K;              // halving steps
    static constexpr int FINAL = ITER >> NH;                // slots left per lane
    static constexpr int PLAIN = K - NH;                    // plain butterfly steps

    static __device__ __forceinline__ int halving_index(int lane) {
        return NH == 0 ? 0 : ((lane & (LPR - 1)) >> PLAIN) & ((1 << NH) - 1);
    }
    // lanes that write the finished sums (the others hold copies)
    static __device__ __forceinline__ bool writer(int lane) {
        return (lane & ((1 << PLAIN) - 1)) == 0;
    }

    template <int WM>
    static __device__ __forceinline__ void run(float (&v)[ITER][WM], int lane) {
#pragma unroll
        for (int s = 0; s < NH; ++s) {
            const int bit = K - 1 - s;
            const int half = ITER >> (s + 1);
            const bool upper = (lane >> bit) & 1;
            // bitwise selects: a select between two elements of v can be
            // rewritten into a load at a selected index, which sends v to
            // scratch memory
            const uint32_t mk = upper ? 0xffffffffu : 0u;
#pragma unroll
            for (int e = 0; e < half; ++e) {
#pragma unroll
                for (int w = 0; w < WM; ++w) {
                    const uint32_t lo = __float_as_uint(v[e][w]), hi = __float_as_uint(v[e + half][w]);
                    const float keep = __uint_as_float((hi & mk) | (lo & ~mk));
                    const float send = __uint_as_float((lo & mk) | (hi & ~mk));
                    v[e][w] = keep + lane_partner(send, bit);
                }
            }
        }
#pragma unroll
        for (int s = 0; s < PLAIN; ++s) {
            const int bit = PLAIN - 1 - s;
#pragma unroll
            for (int w = 0; w < WM; ++w) v[0][w] += lane_partner(v[0][w], bit);
        }
    }
};

// A lane's partial sum of one state row against one query: its PPL float32
// pieces of the row dotted with the query's matching pieces, piece by piece
// and element by element.  Every kernel whose row sums must agree bit for bit
// forms them with this one function.
template <int PPL>
__device__ __forceinline__ float pieces_dot(const f32x4 (&x)[PPL], const f32x4 (&q)[PPL]) {
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < PPL; ++u) {
        acc = fmaf(x[u].x, q[u].x, acc);
        acc = fmaf(x[u].y, q[u].y, acc);
        acc = fmaf(x[u].z, q[u].z, acc);
        acc = fmaf(x[u].w, q[u].w, acc);
    }
    return acc;
}

// Lanes of one wavefront exchanging data through LDS, with no workgroup
// barrier: every lane's writes must come before any lane's reads.  Program
// order alone does not give that, since the compiler may split the
// wavefront at a divergent branch ahead of the exchange and run the rest
// once per subset of lanes (the subset that runs first then reads the other
// subset's stale data).  The wave barrier is convergent, so all lanes meet
// it; the fences keep the LDS accesses on their side of it (within a
// wavefront they need no wait instruction).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// ---- barriers -------------------------------------------------------------
// Workgroup barrier that publishes LDS only.  __syncthreads() also waits for
// every outstanding global store and atomic of the arriving wavefronts; where
// those need not be visible inside the workgroup, this one lets them finish
// in the background.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- per-sequence error bits ----------------------------------------------
__device__ __forceinline__ void raise_seq_error(int32_t *err, int b, int bits) {
    atomicOr(err, bits);
    atomicOr(err + 1 + b, bits);
}

}  // namespace replay
