// qar_device.h -- device-side building blocks of libqar's gfx950 kernels.
//
// Work decomposition shared by every kernel: a lane owns 16 consecutive
// elements (one 16-byte vector of one-byte codes), a 256-thread workgroup owns a
// tile of 4096 elements, and a block of B elements is B/16 adjacent lanes
// (4, 8 or 16) inside one DPP row of a wavefront.  Blocks never straddle
// lanes, wavefronts or tiles, so a block's absmax is a reduction over its
// lanes with DPP row operations and needs neither LDS nor a barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace qar {

constexpr int kLaneElems = 16;
constexpr int kThreads = 256;
constexpr int kTileElems = kLaneElems * kThreads;

// ---------------------------------------------------------------------------
// memory

// Every element, code and dequantized value is touched exactly once, so the
// streams use non-temporal 16-byte accesses (measured on MI355X: about 10%
// more bandwidth than cached ones for these access patterns).  Scales, which
// several lanes share, use ordinary loads and stores.
typedef unsigned int qar_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_b128(const void* p) {
    const qar_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const qar_u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_b128(void* p, uint4 q) {
    const qar_u32x4 v = {q.x, q.y, q.z, q.w};
    __builtin_nontemporal_store(v, reinterpret_cast<qar_u32x4*>(p));
}

typedef unsigned int qar_u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint2 load_b64(const void* p) {
    const qar_u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const qar_u32x2*>(p));
    return make_uint2(v.x, v.y);
}

__device__ __forceinline__ void store_b64(void* p, uint2 q) {
    const qar_u32x2 v = {q.x, q.y};
    __builtin_nontemporal_store(v, reinterpret_cast<qar_u32x2*>(p));
}

__device__ __forceinline__ uint32_t load_b32(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

__device__ __forceinline__ void store_b32(void* p, uint32_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}

__device__ __forceinline__ uint32_t load_b16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
}

__device__ __forceinline__ void store_b16(void* p, uint32_t v) {
    __builtin_nontemporal_store((uint16_t)v, reinterpret_cast<uint16_t*>(p));
}

// ---------------------------------------------------------------------------
// tile order across the chip's eight XCDs
//
// Workgroups are dispatched round-robin over the 8 XCDs (workgroup w goes to
// XCD w % 8).  Renumbering tiles so that each XCD walks one contiguous range
// keeps each XCD's L2 and the DRAM pages it opens on neighbouring addresses.
// The map is a bijection of [0, G) for any grid size G.
__device__ __forceinline__ uint32_t xcd_tile(uint32_t b, uint32_t G) {
    const uint32_t per = G / 8, rem = G % 8, x = b % 8, local = b / 8;
    return x < rem ? x * (per + 1) + local : rem * (per + 1) + (x - rem) * per + local;
}

// The same with super-tiles of S consecutive tiles dealt round-robin to the
// XCDs (S = 0: the contiguous ranges above).  A bijection of [0, G) when
// G % (8 S) == 0, which the launcher guarantees before it passes S > 0.
__device__ __forceinline__ uint32_t xcd_super_tile(uint32_t b, uint32_t G, uint32_t S) {
    if (S == 0) return xcd_tile(b, G);
    const uint32_t x = b % 8, l = b / 8;
    return ((l / S) * 8 + x) * S + l % S;
}

// Which tiles one launch of the reduce computes.  A whole reduce (count 1)
// takes tiles 0 .. ntiles-1 in the XCD order above (super-tiles of `super`,
// 0: ranges).  Chunk `chunk` of `count` interleaved chunks takes runs of q
// consecutive tiles, runs chunk, chunk + count, ...: its local tile t is
// tile ((t / q) count + chunk) q + t % q, taken in dispatch order.
struct TileMap {
    uint32_t super, chunk, count, q;
    __device__ __forceinline__ uint32_t first(uint32_t b, uint32_t G) const {
        return count > 1 ? b : xcd_super_tile(b, G, super);
    }
    __device__ __forceinline__ uint32_t tile(uint32_t t) const {
        return count > 1 ? ((t / q) * count + chunk) * q + t % q : t;
    }
};

// ---------------------------------------------------------------------------
// cross-lane absmax inside a block (DPP row operations, all lanes active)

template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

constexpr int kDppSwapAdjacent = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppSwapPairs = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7-i within each 8 lanes
constexpr int kDppRowMirror = 0x140;     // lane i <-> 15-i within each 16 lanes

// Max over each aligned group of L lanes (4 .. 64); every lane of a group
// gets its group's max.  Up to 16 lanes the groups lie inside one DPP row;
// 32 and 64 lanes add cross-row exchanges.
template <int L>
__device__ __forceinline__ float lanes_max(float m) {
    static_assert(L == 4 || L == 8 || L == 16 || L == 32 || L == 64, "lane group");
    m = fmaxf(m, dpp_move<kDppSwapAdjacent>(m));
    m = fmaxf(m, dpp_move<kDppSwapPairs>(m));
    if constexpr (L >= 8) m = fmaxf(m, dpp_move<kDppRowHalfMirror>(m));
    if constexpr (L >= 16) m = fmaxf(m, dpp_move<kDppRowMirror>(m));
    if constexpr (L >= 32) m = fmaxf(m, __shfl_xor(m, 16));
    if constexpr (L >= 64) m = fmaxf(m, __shfl_xor(m, 32));
    return m;
}

// Max over the B/16 lanes of one block; every lane of the block gets it.
template <int B>
__device__ __forceinline__ float block_max(float m) {
    static_assert(B == 64 || B == 128 || B == 256, "block size");
    return lanes_max<B / kLaneElems>(m);
}

// ---------------------------------------------------------------------------
// element conversions

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

typedef float qar_float2 __attribute__((ext_vector_type(2)));
typedef __bf16 qar_bf16x2 __attribute__((ext_vector_type(2)));

// Two binary32 values -> two bf16, round-to-nearest-even (one
// v_cvt_pk_bf16_f32 on gfx950), packed lo | hi << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const qar_float2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, qar_bf16x2));
}

// Signed code k (0..3) of a packed word, as float.
__device__ __forceinline__ float code_f32(uint32_t w, int k) {
    return (float)(int8_t)(w >> (8 * k));
}

// ---------------------------------------------------------------------------
// quantization of one lane's 16 values with its block's scale s

// Adding 1.5 * 2^23 to a value in [-127, 127] leaves a sum in [2^23, 2^24),
// where the spacing is 1: the addition rounds the value to an integer, ties
// to even (1.5 * 2^23 is even), and the low byte of the sum's bit pattern is
// that integer in two's complement.
constexpr float kRoundMagic = 12582912.0f;

// The quotient x / s, correctly rounded, is computed from the block's
// reciprocal r = 1/s (one IEEE division per lane) and one FMA correction:
//   y = x*r;  e = fma(-y, s, x);  y = fma(e, r, y).
// This equals the IEEE quotient for every pair of binary32 significands:
// tests/test_gpu_quotient_exhaustive.py runs this function on all
// 2^23 x 2^23 pairs and checks each result exactly in binary64 integer
// arithmetic.  Scaling x and s by powers of two scales every intermediate
// alike as long as none of them leaves the normal range, so the identity
// holds for every exponent pair whose intermediates stay normal.  For
// s >= 2^-100 (s never exceeds FLT_MAX/127 < 2^121) r, y and every
// remainder that matters are normal or exact, and a quotient below 1/4 in
// magnitude, whose code is 0 either way, stays below 1/2
// (tests/test_quotient_exponents.py checks both on sampled pairs against
// exact rationals, down to the threshold).  Smaller scales take the IEEE
// division.
constexpr float kFastQuotientMinScale = 0x1p-100f;

__device__ __forceinline__ float fast_quotient(float x, float s, float r) {
    const float y = x * r;
    const float e = __builtin_fmaf(-y, s, x);
    return __builtin_fmaf(e, r, y);
}

// On the fast path the clamp to [-Q, Q] can never change a code, so it is
// left out there.  s = fl(m/Q) is normal, hence s >= (m/Q)(1 - 2^-24), and
// every |x| <= m (m the block's absmax) has |x/s| <= Q/(1 - 2^-24) < Q + 2^-16
// for Q <= 127; Q + 2^-16 is a binary32 value, so the correctly rounded
// quotient is at most Q + 2^-16 and rounds to at most Q.  A subnormal s can
// lie far below m/Q (m = 190 * 2^-149 gives s = 2^-149 and a quotient of
// 190), so the IEEE-division path clamps.
__device__ __forceinline__ uint32_t code_bits_of(float t) { // |t| < 127.5
    return __builtin_bit_cast(uint32_t, t + kRoundMagic);
}

__device__ __forceinline__ uint32_t clamped_code_bits_of(float t) {
    return code_bits_of(__builtin_amdgcn_fmed3f(t, -127.0f, 127.0f));
}

__device__ __forceinline__ uint32_t pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return (a & 0xFFu) | ((b & 0xFFu) << 8) | ((c & 0xFFu) << 16) | (d << 24);
}

// Codes of v[0..15] for scale s; all zero when s == 0.  w[i] receives the
// code of v[i] in its low byte (and 1.5 * 2^23 + code as a float).
// Code bits of P values for an integer code format with largest code Q
// (as quantize16 below, for any count): w[i] holds 1.5 * 2^23 + code_i as a
// float, its low bits the code in two's complement.
template <int P>
__device__ __forceinline__ void int_code_words(const float (&v)[P], float s, float q, uint32_t (&w)[P]) {
    if (s >= kFastQuotientMinScale) {
        const float r = 1.0f / s;
#pragma unroll
        for (int i = 0; i < P; ++i) w[i] = code_bits_of(fast_quotient(v[i], s, r));
    } else if (s != 0.0f) {
#pragma unroll
        for (int i = 0; i < P; ++i)
            w[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_fmed3f(v[i] / s, -q, q) + kRoundMagic);
    } else {
#pragma unroll
        for (int i = 0; i < P; ++i) w[i] = __builtin_bit_cast(uint32_t, kRoundMagic);
    }
}

__device__ __forceinline__ uint4 quantize16(const float (&v)[kLaneElems], float s,
                                            uint32_t (&w)[kLaneElems]) {
    if (s >= kFastQuotientMinScale) {
        const float r = 1.0f / s;
#pragma unroll
        for (int i = 0; i < kLaneElems; ++i) w[i] = code_bits_of(fast_quotient(v[i], s, r));
    } else if (s != 0.0f) {
#pragma unroll
        for (int i = 0; i < kLaneElems; ++i) w[i] = clamped_code_bits_of(v[i] / s);
    } else {
#pragma unroll
        for (int i = 0; i < kLaneElems; ++i) w[i] = __builtin_bit_cast(uint32_t, kRoundMagic);
    }
    uint4 q;
    q.x = pack4(w[0], w[1], w[2], w[3]);
    q.y = pack4(w[4], w[5], w[6], w[7]);
    q.z = pack4(w[8], w[9], w[10], w[11]);
    q.w = pack4(w[12], w[13], w[14], w[15]);
    return q;
}

__device__ __forceinline__ uint4 quantize16(const float (&v)[kLaneElems], float s) {
    uint32_t w[kLaneElems];
    return quantize16(v, s, w);
}

// Dequantized values of the codes held in w[] (as produced by quantize16):
// (w - 1.5*2^23) recovers the code exactly as a float.
__device__ __forceinline__ void dequantize_words(const uint32_t (&w)[kLaneElems], float s,
                                                 float (&y)[kLaneElems]) {
#pragma unroll
    for (int i = 0; i < kLaneElems; ++i) y[i] = (__builtin_bit_cast(float, w[i]) - kRoundMagic) * s;
}

__device__ __forceinline__ float lane_absmax(const float (&v)[kLaneElems]) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < kLaneElems; ++i) m = fmaxf(m, fabsf(v[i]));
    return m;
}

// y_i = (float)q_i * s for the 16 codes of a lane
__device__ __forceinline__ void dequantize16(uint4 q, float s, float (&y)[kLaneElems]) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) y[4 * j + k] = code_f32(w[j], k) * s;
}

// ---------------------------------------------------------------------------
// code formats.  A policy gives Q_max (the value a block's absmax maps to),
// the type of a lane's 16 codes (Vec) and how to load, store, make and read
// them.  Byte-wide formats (int8, E4M3) keep a lane's codes in one 16-byte
// vector at byte offset e0; the 4-bit format packs them into 8 bytes at e0/2.
// scaled8/scaled4 give code * s (one binary32 product each) for the 8 or 4
// consecutive elements starting at e (a multiple of 8 or 4), their codes
// read from global memory or LDS, for the kernels that write their output
// in contiguous 16-byte slots.

// EQuARX's integers: q = clamp(rne(x/s), -127, 127), s = absmax / 127.
struct Int8Codes {
    using Vec = uint4;
    static constexpr float kQmax = 127.0f;
    static __device__ __forceinline__ size_t bytes(size_t e) { return e; }
    static __device__ __forceinline__ Vec load(const int8_t* c, size_t e0) { return load_b128(c + e0); }
    static __device__ __forceinline__ void store(int8_t* c, size_t e0, Vec q) { store_b128(c + e0, q); }
    static __device__ __forceinline__ float value(uint32_t w, int k) { return code_f32(w, k); }
    static __device__ __forceinline__ Vec quantize(const float (&v)[kLaneElems], float s) {
        return quantize16(v, s);
    }
    static __device__ __forceinline__ void dequantize(Vec q, float s, float (&y)[kLaneElems]) {
        dequantize16(q, s, y);
    }
    static __device__ __forceinline__ void scaled8(const int8_t* c, size_t e, float s, float (&y)[8]) {
        const uint2 w = *reinterpret_cast<const uint2*>(c + e);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            y[k] = value(w.x, k) * s;
            y[4 + k] = value(w.y, k) * s;
        }
    }
    static __device__ __forceinline__ void scaled4(const int8_t* c, size_t e, float s, float (&y)[4]) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(c + e);
#pragma unroll
        for (int k = 0; k < 4; ++k) y[k] = value(w, k) * s;
    }
    // P = 8 or 4 consecutive codes from element e (a multiple of P): 8 or 4
    // bytes, for the kernels whose lanes own P-element slots of data
    template <int P>
    using Pack = std::conditional_t<P == 8, uint2, uint32_t>;
    template <int P>
    static __device__ __forceinline__ Pack<P> load_p(const int8_t* c, size_t e) {
        if constexpr (P == 8) return load_b64(c + e);
        else return load_b32(c + e);
    }
    template <int P>
    static __device__ __forceinline__ void store_p(int8_t* c, size_t e, Pack<P> q) {
        if constexpr (P == 8) store_b64(c + e, q);
        else store_b32(c + e, q);
    }
    template <int P>
    static __device__ __forceinline__ Pack<P> quantize_p(const float (&v)[P], float s) {
        uint32_t w[P];
        int_code_words<P>(v, s, kQmax, w);
        if constexpr (P == 8) return make_uint2(pack4(w[0], w[1], w[2], w[3]), pack4(w[4], w[5], w[6], w[7]));
        else return pack4(w[0], w[1], w[2], w[3]);
    }
    template <int P>
    static __device__ __forceinline__ void dequantize_p(Pack<P> q, float s, float (&y)[P]) {
        if constexpr (P == 8) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                y[k] = value(q.x, k) * s;
                y[4 + k] = value(q.y, k) * s;
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) y[k] = value(q, k) * s;
        }
    }
};

// FP8 E4M3 in the OCP format (bias 7, 3 mantissa bits, no infinity, largest
// finite 448), the format the TACO page argues for: s = absmax / 448 and the
// code is the E4M3 value nearest to fl32(x / s) clamped to [-448, 448], ties
// to even, sign kept.  gfx950's v_cvt_pk_fp8_f32 rounds to nearest even into
// this format and v_cvt_f32_fp8 widens exactly.
//
// The quotient is the same exact FMA-corrected one as for int8, with a
// higher threshold: quotients down to 2^-10 decide a code here (smaller
// ones give +-0 with the sign of x), and for a quotient y >= 2^-11 the
// remainder x - y*s is a multiple of 2^(-11-23) * 2^(-90-23) >= 2^-149, so
// exact, when s >= 2^-90.  The FMA correction keeps a nonzero quotient's
// sign; only x = -0 needs its sign restored.
struct E4M3Codes {
    using Vec = uint4;
    static constexpr float kQmax = 448.0f;
    static __device__ __forceinline__ size_t bytes(size_t e) { return e; }
    static __device__ __forceinline__ Vec load(const int8_t* c, size_t e0) { return load_b128(c + e0); }
    static __device__ __forceinline__ void store(int8_t* c, size_t e0, Vec q) { store_b128(c + e0, q); }
    static constexpr float kFastMinScale = 0x1p-90f;
    static __device__ __forceinline__ float value(uint32_t w, int k) {
        switch (k) {
        case 0: return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
        case 1: return __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
        case 2: return __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
        default: return __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
        }
    }
    // Four quotients of magnitude at most 448 + 2^-15 into four codes.  The
    // conversion rounds 448 + 2^-15 to 448 (0x7E) but turns anything from 465
    // up into NaN (0x7F), so larger quotients must be clamped first.
    static __device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
        return (uint32_t)w;
    }
    // the quotients of P values, ready for conversion (s != 0)
    template <int P>
    static __device__ __forceinline__ void quotients(const float (&v)[P], float s, float (&t)[P]) {
        if (s >= kFastMinScale) {
            const float r = 1.0f / s;
#pragma unroll
            for (int i = 0; i < P; ++i) {
                // x = -0 gives e = +0 and +0 + -0 = +0: put the sign back.
                // No clamp: as for int8 (code_bits_of), a normal s bounds the
                // rounded quotient by Q + 2^-15 here.
                t[i] = __builtin_copysignf(fast_quotient(v[i], s, r), v[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < P; ++i) t[i] = __builtin_amdgcn_fmed3f(v[i] / s, -kQmax, kQmax);
        }
    }
    static __device__ __forceinline__ uint4 quantize(const float (&v)[kLaneElems], float s) {
        if (s == 0.0f) return make_uint4(0u, 0u, 0u, 0u);
        float t[kLaneElems];
        quotients<kLaneElems>(v, s, t);
        uint4 q;
        q.x = pack4(t[0], t[1], t[2], t[3]);
        q.y = pack4(t[4], t[5], t[6], t[7]);
        q.z = pack4(t[8], t[9], t[10], t[11]);
        q.w = pack4(t[12], t[13], t[14], t[15]);
        return q;
    }
    static __device__ __forceinline__ void dequantize(uint4 q, float s, float (&y)[kLaneElems]) {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int k = 0; k < 4; ++k) y[4 * j + k] = value(w[j], k) * s;
    }
    static __device__ __forceinline__ void scaled8(const int8_t* c, size_t e, float s, float (&y)[8]) {
        const uint2 w = *reinterpret_cast<const uint2*>(c + e);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            y[k] = value(w.x, k) * s;
            y[4 + k] = value(w.y, k) * s;
        }
    }
    static __device__ __forceinline__ void scaled4(const int8_t* c, size_t e, float s, float (&y)[4]) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(c + e);
#pragma unroll
        for (int k = 0; k < 4; ++k) y[k] = value(w, k) * s;
    }
    // P = 8 or 4 consecutive codes (as Int8Codes)
    template <int P>
    using Pack = std::conditional_t<P == 8, uint2, uint32_t>;
    template <int P>
    static __device__ __forceinline__ Pack<P> load_p(const int8_t* c, size_t e) {
        if constexpr (P == 8) return load_b64(c + e);
        else return load_b32(c + e);
    }
    template <int P>
    static __device__ __forceinline__ void store_p(int8_t* c, size_t e, Pack<P> q) {
        if constexpr (P == 8) store_b64(c + e, q);
        else store_b32(c + e, q);
    }
    template <int P>
    static __device__ __forceinline__ Pack<P> quantize_p(const float (&v)[P], float s) {
        if (s == 0.0f) return Pack<P>{};
        float t[P];
        quotients<P>(v, s, t);
        if constexpr (P == 8) return make_uint2(pack4(t[0], t[1], t[2], t[3]), pack4(t[4], t[5], t[6], t[7]));
        else return pack4(t[0], t[1], t[2], t[3]);
    }
    template <int P>
    static __device__ __forceinline__ void dequantize_p(Pack<P> q, float s, float (&y)[P]) {
        if constexpr (P == 8) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                y[k] = value(q.x, k) * s;
                y[4 + k] = value(q.y, k) * s;
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) y[k] = value(q, k) * s;
        }
    }
};

// 4-bit integers, the int8 rules at 4 bits: q = clamp(rne(x/s), -7, 7),
// s = absmax / 7, two codes per byte (element 2k in the low nibble of byte
// k).  The quotient and the rounding are the int8 ones (quotients below 1/4
// give code 0 either way); the low nibble of the rounded word is the code in
// two's complement.
struct Int4Codes {
    using Vec = uint2;
    static constexpr float kQmax = 7.0f;
    static __device__ __forceinline__ size_t bytes(size_t e) { return e / 2; }
    static __device__ __forceinline__ Vec load(const int8_t* c, size_t e0) { return load_b64(c + e0 / 2); }
    static __device__ __forceinline__ void store(int8_t* c, size_t e0, Vec q) { store_b64(c + e0 / 2, q); }
    // code k (0..7) of a word of 8 nibbles, as float
    static __device__ __forceinline__ float value(uint32_t w, int k) {
        return (float)((int32_t)(w << (28 - 4 * k)) >> 28);
    }
    static __device__ __forceinline__ uint32_t nibbles8(const uint32_t* w) {
        uint32_t r = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) r |= (w[k] & 0xFu) << (4 * k);
        return r;
    }
    static __device__ __forceinline__ Vec quantize(const float (&v)[kLaneElems], float s) {
        uint32_t w[kLaneElems];
        if (s >= kFastQuotientMinScale) {
            const float r = 1.0f / s;
#pragma unroll
            for (int i = 0; i < kLaneElems; ++i) // no clamp needed (see code_bits_of)
                w[i] = __builtin_bit_cast(uint32_t, fast_quotient(v[i], s, r) + kRoundMagic);
        } else if (s != 0.0f) {
#pragma unroll
            for (int i = 0; i < kLaneElems; ++i)
                w[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_fmed3f(v[i] / s, -kQmax, kQmax) + kRoundMagic);
        } else {
            return make_uint2(0u, 0u);
        }
        return make_uint2(nibbles8(w), nibbles8(w + 8));
    }
    // code / 16 for the low nibble of byte BYTE of w: v_cvt_off_f32_i4 maps
    // a 4-bit two's complement integer i to i/16, exactly; the SDWA byte
    // select picks the nibble, so a code costs one instruction
    template <int BYTE>
    static __device__ __forceinline__ float sixteenth(uint32_t w) {
        float f;
        if constexpr (BYTE == 0)
            asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(f) : "v"(w));
        else if constexpr (BYTE == 1)
            asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(f) : "v"(w));
        else if constexpr (BYTE == 2)
            asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(f) : "v"(w));
        else
            asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(f) : "v"(w));
        return f;
    }
    static __device__ __forceinline__ void dequantize8(uint32_t w, float s16, float* y) {
        const uint32_t hi = w >> 4; // odd codes into the low nibbles
        y[0] = sixteenth<0>(w) * s16;
        y[1] = sixteenth<0>(hi) * s16;
        y[2] = sixteenth<1>(w) * s16;
        y[3] = sixteenth<1>(hi) * s16;
        y[4] = sixteenth<2>(w) * s16;
        y[5] = sixteenth<2>(hi) * s16;
        y[6] = sixteenth<3>(w) * s16;
        y[7] = sixteenth<3>(hi) * s16;
    }
    // y = code * s.  For s <= 2^123, (code/16) * (16 s) is the same real
    // product (16 s is exact and finite), so it rounds to the same binary32
    // value, signed zeros included; larger, infinite or NaN scales take the
    // integer conversion.
    static __device__ __forceinline__ void dequantize(Vec q, float s, float (&y)[kLaneElems]) {
        if (s <= 0x1p123f) {
            const float s16 = s * 16.0f;
            dequantize8(q.x, s16, y);
            dequantize8(q.y, s16, y + 8);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                y[k] = value(q.x, k) * s;
                y[8 + k] = value(q.y, k) * s;
            }
        }
    }
    // the same products for 8 or 4 codes (4 or 2 bytes), widened as in dequantize
    static __device__ __forceinline__ void scaled8(const int8_t* c, size_t e, float s, float (&y)[8]) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(c + e / 2);
        if (s <= 0x1p123f) {
            dequantize8(w, s * 16.0f, y);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) y[k] = value(w, k) * s;
        }
    }
    static __device__ __forceinline__ void scaled4(const int8_t* c, size_t e, float s, float (&y)[4]) {
        const uint32_t w = *reinterpret_cast<const uint16_t*>(c + e / 2);
        if (s <= 0x1p123f) {
            const float s16 = s * 16.0f;
            const uint32_t hi = w >> 4; // codes 1 and 3 into the low nibbles of bytes 0 and 1
            y[0] = sixteenth<0>(w) * s16;
            y[1] = sixteenth<0>(hi) * s16;
            y[2] = sixteenth<1>(w) * s16;
            y[3] = sixteenth<1>(hi) * s16;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) y[k] = value(w, k) * s;
        }
    }
    // P = 8 or 4 consecutive codes from element e (a multiple of P): 4 or 2
    // bytes at e / 2, in the low bits of a word
    template <int P>
    using Pack = uint32_t;
    template <int P>
    static __device__ __forceinline__ uint32_t load_p(const int8_t* c, size_t e) {
        if constexpr (P == 8) return load_b32(c + e / 2);
        else return load_b16(c + e / 2);
    }
    template <int P>
    static __device__ __forceinline__ void store_p(int8_t* c, size_t e, uint32_t q) {
        if constexpr (P == 8) store_b32(c + e / 2, q);
        else store_b16(c + e / 2, q);
    }
    template <int P>
    static __device__ __forceinline__ uint32_t quantize_p(const float (&v)[P], float s) {
        uint32_t w[P];
        int_code_words<P>(v, s, kQmax, w);
        uint32_t r = 0;
#pragma unroll
        for (int k = 0; k < P; ++k) r |= (w[k] & 0xFu) << (4 * k);
        return r;
    }
    template <int P>
    static __device__ __forceinline__ void dequantize_p(uint32_t q, float s, float (&y)[P]) {
        if constexpr (P == 8) {
            if (s <= 0x1p123f) {
                dequantize8(q, s * 16.0f, y);
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) y[k] = value(q, k) * s;
            }
        } else {
            if (s <= 0x1p123f) {
                const float s16 = s * 16.0f;
                const uint32_t hi = q >> 4; // codes 1 and 3 into the low nibbles of bytes 0 and 1
                y[0] = sixteenth<0>(q) * s16;
                y[1] = sixteenth<0>(hi) * s16;
                y[2] = sixteenth<1>(q) * s16;
                y[3] = sixteenth<1>(hi) * s16;
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) y[k] = value(q, k) * s;
            }
        }
    }
};

// ---------------------------------------------------------------------------
// lane loads and stores of element data

// A lane's 16 elements as loaded (32 bytes of bf16 or 64 of fp32), so a
// caller can put other loads in flight before it converts them.
template <typename In>
struct Raw16 {
    static constexpr int kWords = kLaneElems * (int)sizeof(In) / 16;
    uint4 w[kWords];
};

template <typename In>
__device__ __forceinline__ Raw16<In> load_raw16(const In* p) {
    Raw16<In> r;
#pragma unroll
    for (int j = 0; j < Raw16<In>::kWords; ++j) r.w[j] = load_b128(p + j * (16 / sizeof(In)));
    return r;
}

__device__ __forceinline__ void unpack16(const Raw16<uint16_t>& r, float (&v)[kLaneElems]) {
    const uint32_t w[8] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w, r.w[1].x, r.w[1].y, r.w[1].z, r.w[1].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        v[2 * j] = bf16_lo(w[j]);
        v[2 * j + 1] = bf16_hi(w[j]);
    }
}

__device__ __forceinline__ void unpack16(const Raw16<float>& r, float (&v)[kLaneElems]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[4 * j + 0] = __builtin_bit_cast(float, r.w[j].x);
        v[4 * j + 1] = __builtin_bit_cast(float, r.w[j].y);
        v[4 * j + 2] = __builtin_bit_cast(float, r.w[j].z);
        v[4 * j + 3] = __builtin_bit_cast(float, r.w[j].w);
    }
}

template <typename In>
__device__ __forceinline__ void load16(const In* p, float (&v)[kLaneElems]) {
    unpack16(load_raw16(p), v);
}

__device__ __forceinline__ void store16(uint16_t* p, const float (&v)[kLaneElems]) {
    uint4 a, b;
    a.x = pack_bf16x2(v[0], v[1]);
    a.y = pack_bf16x2(v[2], v[3]);
    a.z = pack_bf16x2(v[4], v[5]);
    a.w = pack_bf16x2(v[6], v[7]);
    b.x = pack_bf16x2(v[8], v[9]);
    b.y = pack_bf16x2(v[10], v[11]);
    b.z = pack_bf16x2(v[12], v[13]);
    b.w = pack_bf16x2(v[14], v[15]);
    store_b128(p, a);
    store_b128(p + 8, b);
}

__device__ __forceinline__ void store16(float* p, const float (&v)[kLaneElems]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint4 a;
        a.x = __builtin_bit_cast(uint32_t, v[4 * j + 0]);
        a.y = __builtin_bit_cast(uint32_t, v[4 * j + 1]);
        a.z = __builtin_bit_cast(uint32_t, v[4 * j + 2]);
        a.w = __builtin_bit_cast(uint32_t, v[4 * j + 3]);
        store_b128(p + 4 * j, a);
    }
}

} // namespace qar
