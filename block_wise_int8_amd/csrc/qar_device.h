// qar_device.h -- device-side building blocks of libqar's gfx950 kernels.
//
// Work decomposition shared by every kernel: a lane owns 16 consecutive
// elements (one 16-byte vector of int8 codes), a 256-thread workgroup owns a
// tile of 4096 elements, and a block of B elements is B/16 adjacent lanes
// (4, 8 or 16) inside one DPP row of a wavefront.  Blocks never straddle
// lanes, wavefronts or tiles, so a block's absmax is a reduction over its
// lanes with DPP row operations and needs neither LDS nor a barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qar {

constexpr int kLaneElems = 16;
constexpr int kThreads = 256;
constexpr int kTileElems = kLaneElems * kThreads;

// ---------------------------------------------------------------------------
// memory

__device__ __forceinline__ uint4 load_b128(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ void store_b128(void* p, uint4 v) {
    *reinterpret_cast<uint4*>(p) = v;
}

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

// Max over the B/16 lanes of one block; every lane of the block gets it.
template <int B>
__device__ __forceinline__ float block_max(float m) {
    static_assert(B == 64 || B == 128 || B == 256, "block size");
    m = fmaxf(m, dpp_move<kDppSwapAdjacent>(m));
    m = fmaxf(m, dpp_move<kDppSwapPairs>(m));
    if constexpr (B >= 128) m = fmaxf(m, dpp_move<kDppRowHalfMirror>(m));
    if constexpr (B >= 256) m = fmaxf(m, dpp_move<kDppRowMirror>(m));
    return m;
}

// ---------------------------------------------------------------------------
// element conversions

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Round-to-nearest-even of a binary32 value to bf16 (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return bf16_rne(lo) | (bf16_rne(hi) << 16);
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

__device__ __forceinline__ uint32_t code_word(float x, float s) {
    float t = x / s; // correctly rounded binary32 division
    t = __builtin_amdgcn_fmed3f(t, -127.0f, 127.0f);
    return __builtin_bit_cast(uint32_t, t + kRoundMagic);
}

__device__ __forceinline__ uint32_t pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return (a & 0xFFu) | ((b & 0xFFu) << 8) | ((c & 0xFFu) << 16) | (d << 24);
}

// Codes of v[0..15] for scale s; all zero when s == 0.
__device__ __forceinline__ uint4 quantize16(const float (&v)[kLaneElems], float s) {
    uint32_t w[kLaneElems];
#pragma unroll
    for (int i = 0; i < kLaneElems; ++i) w[i] = code_word(v[i], s);
    uint4 q;
    q.x = pack4(w[0], w[1], w[2], w[3]);
    q.y = pack4(w[4], w[5], w[6], w[7]);
    q.z = pack4(w[8], w[9], w[10], w[11]);
    q.w = pack4(w[12], w[13], w[14], w[15]);
    if (s == 0.0f) q = make_uint4(0u, 0u, 0u, 0u);
    return q;
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
// lane loads and stores of element data

__device__ __forceinline__ void load16(const uint16_t* p, float (&v)[kLaneElems]) {
    uint4 a = load_b128(p);
    uint4 b = load_b128(p + 8);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        v[2 * j] = bf16_lo(w[j]);
        v[2 * j + 1] = bf16_hi(w[j]);
    }
}

__device__ __forceinline__ void load16(const float* p, float (&v)[kLaneElems]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint4 a = load_b128(p + 4 * j);
        v[4 * j + 0] = __builtin_bit_cast(float, a.x);
        v[4 * j + 1] = __builtin_bit_cast(float, a.y);
        v[4 * j + 2] = __builtin_bit_cast(float, a.z);
        v[4 * j + 3] = __builtin_bit_cast(float, a.w);
    }
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
