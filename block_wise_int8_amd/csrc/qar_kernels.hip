// qar_kernels.hip -- libqar's gfx950 kernels and their launchers.
//
// Method: EQuARX ("EQuARX: Efficient Quantized AllReduce in XLA for
// Distributed Machine Learning Acceleration"), page summary, section
// "technical framework": blocks (step 1), dynamic per-block quantization to
// INT8 (step 2, with the run-time range of "key design" item 1), reduction of
// quantized contributions (step 3), dequantization (step 4).  The arithmetic
// each kernel performs is spelled out in include/qar.h.
//
// Every kernel streams HBM once: 16-byte loads and stores per lane, a block's
// absmax by DPP inside its lanes, the requantization fused behind the
// reduction so the fp32 sum never leaves registers.  A workgroup walks tiles
// of 4096 elements with a grid-stride loop (the grid is capped, the loop
// covers any n).
#include "qar_device.h"
#include "qar_launch.h"

namespace qar {

// ---------------------------------------------------------------------------
// quantize: x (bf16 or fp32) -> codes, scales

template <int B, typename In>
__global__ __launch_bounds__(kThreads) void k_quantize(const In* __restrict__ x, size_t n,
                                                       int8_t* __restrict__ codes,
                                                       float* __restrict__ scales,
                                                       uint32_t ntiles) {
    for (uint32_t tile = xcd_tile(blockIdx.x, gridDim.x); tile < ntiles; tile += gridDim.x) {
        const size_t e0 = ((size_t)tile * kThreads + threadIdx.x) * kLaneElems;
        const bool valid = e0 < n;
        // Lanes past the end read element 0 instead: blocks never straddle
        // the end, so their (discarded) results cannot touch a valid block.
        const size_t ld = valid ? e0 : 0;
        float v[kLaneElems];
        load16(x + ld, v);
        const float s = block_max<B>(lane_absmax(v)) / 127.0f;
        const uint4 q = quantize16(v, s);
        if (valid) {
            store_b128(codes + e0, q);
            if (e0 % B == 0) scales[e0 / B] = s;
        }
    }
}

// ---------------------------------------------------------------------------
// one-shot reduce: N quantized ranks -> requantized sum (+ optional dequant)

// Dequantized output of one wavefront's 1024-element tile, written so that
// every 16-byte store instruction covers contiguous memory (1 KB per
// instruction).  A lane holds 16 consecutive codes (32 bytes of bf16, 64 of
// fp32), so the codes and scales of the wave are staged in LDS and each lane
// reads back the 8 (bf16) or 4 (fp32) codes that belong to its store slots.
// Only lanes of one wavefront exchange data, so a wave barrier suffices.
template <int B, int OUT>
__device__ __forceinline__ void store_dequantized_tile(uint4 qo, float so, size_t e0, size_t n, void* out,
                                                       uint4* lds_codes, float* lds_scales) {
    constexpr int kLanesPerBlock = B / kLaneElems;
    const int lane = threadIdx.x & 63;
    lds_codes[lane] = qo;
    if (lane % kLanesPerBlock == 0) lds_scales[lane / kLanesPerBlock] = so;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const size_t wave0 = e0 - (size_t)lane * kLaneElems; // first element of the wave's tile
    const int8_t* codes = reinterpret_cast<const int8_t*>(lds_codes);
    if constexpr (OUT == kOutBF16) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = 512 * j + 8 * lane; // element within the wave tile
            const uint2 c = *reinterpret_cast<const uint2*>(codes + e);
            const float s = lds_scales[e / B];
            uint4 o;
            o.x = pack_bf16x2(code_f32(c.x, 0) * s, code_f32(c.x, 1) * s);
            o.y = pack_bf16x2(code_f32(c.x, 2) * s, code_f32(c.x, 3) * s);
            o.z = pack_bf16x2(code_f32(c.y, 0) * s, code_f32(c.y, 1) * s);
            o.w = pack_bf16x2(code_f32(c.y, 2) * s, code_f32(c.y, 3) * s);
            if (wave0 + e < n) store_b128(static_cast<uint16_t*>(out) + wave0 + e, o);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 256 * j + 4 * lane;
            const uint32_t c = *reinterpret_cast<const uint32_t*>(codes + e);
            const float s = lds_scales[e / B];
            uint4 o;
            o.x = __builtin_bit_cast(uint32_t, code_f32(c, 0) * s);
            o.y = __builtin_bit_cast(uint32_t, code_f32(c, 1) * s);
            o.z = __builtin_bit_cast(uint32_t, code_f32(c, 2) * s);
            o.w = __builtin_bit_cast(uint32_t, code_f32(c, 3) * s);
            if (wave0 + e < n) store_b128(static_cast<float*>(out) + wave0 + e, o);
        }
    }
    // the next tile overwrites the staging area: keep this tile's reads first
    __builtin_amdgcn_wave_barrier();
}

template <int B, int OUT>
__global__ __launch_bounds__(kThreads) void k_reduce(RankPtrs rp, int nranks, size_t n,
                                                     int8_t* codes_out, float* scales_out,
                                                     void* __restrict__ out, uint32_t ntiles) {
    constexpr int G = 8; // ranks whose loads are in flight together
    __shared__ uint4 lds_codes[OUT != kOutNone ? kThreads : 1];
    __shared__ float lds_scales[OUT != kOutNone ? kThreads * kLaneElems / B : 1];
    for (uint32_t tile = xcd_tile(blockIdx.x, gridDim.x); tile < ntiles; tile += gridDim.x) {
        const size_t e0 = ((size_t)tile * kThreads + threadIdx.x) * kLaneElems;
        const bool valid = e0 < n;
        const size_t ld = valid ? e0 : 0; // see k_quantize
        const size_t blk = ld / B;
        float acc[kLaneElems];
        for (int g = 0; g < nranks; g += G) {
            uint4 q[G];
            float s[G];
#pragma unroll
            for (int j = 0; j < G; ++j) {
                if (g + j < nranks) {
                    q[j] = load_b128(rp.codes[g + j] + ld);
                    s[j] = rp.scales[g + j][blk];
                }
            }
#pragma unroll
            for (int j = 0; j < G; ++j) {
                if (g + j < nranks) {
                    float y[kLaneElems];
                    dequantize16(q[j], s[j], y);
                    if (g + j == 0) {
#pragma unroll
                        for (int i = 0; i < kLaneElems; ++i) acc[i] = y[i];
                    } else {
#pragma unroll
                        for (int i = 0; i < kLaneElems; ++i) acc[i] = acc[i] + y[i];
                    }
                }
            }
        }
        const float so = block_max<B>(lane_absmax(acc)) / 127.0f;
        const uint4 qo = quantize16(acc, so);
        if (valid) {
            store_b128(codes_out + e0, qo);
            if (e0 % B == 0) scales_out[blk] = so;
        }
        if constexpr (OUT != kOutNone) {
            const int wave = threadIdx.x / 64;
            store_dequantized_tile<B, OUT>(qo, so, e0, n, out, lds_codes + wave * 64,
                                           lds_scales + wave * (64 * kLaneElems / B));
        }
    }
}

// ---------------------------------------------------------------------------
// ring step: dequantize incoming + add local (bf16/fp32) + requantize

template <int B, typename In>
__global__ __launch_bounds__(kThreads) void k_ring_step(const int8_t* codes_in, const float* scales_in,
                                                        const In* __restrict__ local, size_t n,
                                                        int8_t* codes_out, float* scales_out,
                                                        uint32_t ntiles) {
    for (uint32_t tile = xcd_tile(blockIdx.x, gridDim.x); tile < ntiles; tile += gridDim.x) {
        const size_t e0 = ((size_t)tile * kThreads + threadIdx.x) * kLaneElems;
        const bool valid = e0 < n;
        const size_t ld = valid ? e0 : 0; // see k_quantize
        const size_t blk = ld / B;
        float acc[kLaneElems];
        {
            const uint4 q = load_b128(codes_in + ld);
            const float s = scales_in[blk];
            float x[kLaneElems];
            load16(local + ld, x);
            dequantize16(q, s, acc);
#pragma unroll
            for (int i = 0; i < kLaneElems; ++i) acc[i] = acc[i] + x[i];
        }
        const float so = block_max<B>(lane_absmax(acc)) / 127.0f;
        const uint4 qo = quantize16(acc, so);
        if (valid) {
            store_b128(codes_out + e0, qo);
            if (e0 % B == 0) scales_out[blk] = so;
        }
    }
}

// ---------------------------------------------------------------------------
// dequantize: codes, scales -> bf16 or fp32

// Each 16-byte store instruction writes 1 KB of contiguous output: lane L of
// a wavefront owns the store slots at elements 8L + 512j (bf16, j = 0..1) or
// 4L + 256j (fp32, j = 0..3) of the wave's 1024-element tile and reads the
// 8 or 4 codes of each slot directly (8 or 4 bytes, 512 or 256 bytes
// contiguous per load instruction).
template <int B, typename Out>
__global__ __launch_bounds__(kThreads) void k_dequantize(const int8_t* __restrict__ codes,
                                                         const float* __restrict__ scales, size_t n,
                                                         Out* __restrict__ out, uint32_t ntiles) {
    constexpr int kSlot = 16 / sizeof(Out);      // elements per 16-byte store
    constexpr int kSlots = kLaneElems / kSlot;   // store slots per lane
    const int lane = threadIdx.x & 63;
    for (uint32_t tile = xcd_tile(blockIdx.x, gridDim.x); tile < ntiles; tile += gridDim.x) {
        const size_t wave0 = ((size_t)tile * kThreads + (threadIdx.x & ~63u)) * kLaneElems;
#pragma unroll
        for (int j = 0; j < kSlots; ++j) {
            const size_t e = wave0 + (size_t)j * 64 * kSlot + (size_t)lane * kSlot;
            if (e >= n) continue; // n % 64 == 0: a slot is wholly inside or outside
            const float s = scales[e / B];
            uint4 o;
            if constexpr (kSlot == 8) {
                const uint2 c = *reinterpret_cast<const uint2*>(codes + e);
                o.x = pack_bf16x2(code_f32(c.x, 0) * s, code_f32(c.x, 1) * s);
                o.y = pack_bf16x2(code_f32(c.x, 2) * s, code_f32(c.x, 3) * s);
                o.z = pack_bf16x2(code_f32(c.y, 0) * s, code_f32(c.y, 1) * s);
                o.w = pack_bf16x2(code_f32(c.y, 2) * s, code_f32(c.y, 3) * s);
            } else {
                const uint32_t c = *reinterpret_cast<const uint32_t*>(codes + e);
                o.x = __builtin_bit_cast(uint32_t, code_f32(c, 0) * s);
                o.y = __builtin_bit_cast(uint32_t, code_f32(c, 1) * s);
                o.z = __builtin_bit_cast(uint32_t, code_f32(c, 2) * s);
                o.w = __builtin_bit_cast(uint32_t, code_f32(c, 3) * s);
            }
            store_b128(out + e, o);
        }
    }
}

// ---------------------------------------------------------------------------
// the unquantized comparator: fp32 rank-order sum of N bf16/fp32 buffers

// No block structure here, so every lane works on contiguous store slots:
// lane L of a wavefront owns the 16-byte slots at elements
// kSlot*L + 64*kSlot*j of the wave's 1024-element tile (kSlot = 8 for bf16,
// 4 for fp32), and every load and store instruction covers 1 KB.
template <typename T>
struct SlotTraits;
template <>
struct SlotTraits<uint16_t> {
    static constexpr int kSlot = 8;
    static constexpr int kGroup = 8; // ranks whose loads are in flight together
    static __device__ __forceinline__ void widen(uint4 w, float* v) {
        const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = bf16_lo(a[k]);
            v[2 * k + 1] = bf16_hi(a[k]);
        }
    }
    static __device__ __forceinline__ uint4 narrow(const float* v) {
        return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                          pack_bf16x2(v[6], v[7]));
    }
};
template <>
struct SlotTraits<float> {
    static constexpr int kSlot = 4;
    static constexpr int kGroup = 4;
    static __device__ __forceinline__ void widen(uint4 w, float* v) {
        v[0] = __builtin_bit_cast(float, w.x);
        v[1] = __builtin_bit_cast(float, w.y);
        v[2] = __builtin_bit_cast(float, w.z);
        v[3] = __builtin_bit_cast(float, w.w);
    }
    static __device__ __forceinline__ uint4 narrow(const float* v) {
        return make_uint4(__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1]),
                          __builtin_bit_cast(uint32_t, v[2]), __builtin_bit_cast(uint32_t, v[3]));
    }
};

template <typename T>
__global__ __launch_bounds__(kThreads) void k_reduce_unquantized(PlainPtrs xp, int nranks, size_t n, T* out,
                                                                 uint32_t ntiles) {
    using S = SlotTraits<T>;
    constexpr int kSlot = S::kSlot, kSlots = kLaneElems / kSlot, G = S::kGroup;
    const int lane = threadIdx.x & 63;
    for (uint32_t tile = xcd_tile(blockIdx.x, gridDim.x); tile < ntiles; tile += gridDim.x) {
        const size_t wave0 = ((size_t)tile * kThreads + (threadIdx.x & ~63u)) * kLaneElems;
        size_t e[kSlots], ld[kSlots];
#pragma unroll
        for (int j = 0; j < kSlots; ++j) {
            e[j] = wave0 + (size_t)j * 64 * kSlot + (size_t)lane * kSlot;
            ld[j] = e[j] < n ? e[j] : 0; // n % 16 == 0: a slot is wholly inside or outside
        }
        float acc[kLaneElems];
        for (int g = 0; g < nranks; g += G) {
            uint4 raw[G][kSlots];
#pragma unroll
            for (int r = 0; r < G; ++r)
                if (g + r < nranks)
#pragma unroll
                    for (int j = 0; j < kSlots; ++j) raw[r][j] = load_b128(static_cast<const T*>(xp.x[g + r]) + ld[j]);
#pragma unroll
            for (int r = 0; r < G; ++r) {
                if (g + r < nranks) {
                    float v[kLaneElems];
#pragma unroll
                    for (int j = 0; j < kSlots; ++j) S::widen(raw[r][j], v + j * kSlot);
                    if (g + r == 0) {
#pragma unroll
                        for (int i = 0; i < kLaneElems; ++i) acc[i] = v[i];
                    } else {
#pragma unroll
                        for (int i = 0; i < kLaneElems; ++i) acc[i] = acc[i] + v[i];
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kSlots; ++j)
            if (e[j] < n) store_b128(out + e[j], S::narrow(acc + j * kSlot));
    }
}

// ---------------------------------------------------------------------------
// row-bounded blocks: a [rows, row_len] tensor whose rows restart the block
// grid, so the last block of a row may be partial (row_len % B elements).
// One wavefront per block; lane l owns the block's elements l, l+64, l+128,
// l+192 (B <= 256).  Elements move one by one (each access instruction is
// still contiguous across the wave); this is the general path, taken only
// when row_len % B != 0.

struct RowMap {
    size_t rows, row_len;
    uint32_t block, per_row; // per_row = ceil(row_len / block)
    __device__ __forceinline__ void locate(size_t b, size_t& start, uint32_t& len) const {
        const size_t r = b / per_row, k = b % per_row;
        const size_t col = k * block;
        start = r * row_len + col;
        len = (uint32_t)(row_len - col < block ? row_len - col : block);
    }
};

__device__ __forceinline__ float wave_max(float m) {
    m = fmaxf(m, dpp_move<kDppSwapAdjacent>(m));
    m = fmaxf(m, dpp_move<kDppSwapPairs>(m));
    m = fmaxf(m, dpp_move<kDppRowHalfMirror>(m));
    m = fmaxf(m, dpp_move<kDppRowMirror>(m));
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    return m;
}

__device__ __forceinline__ float load_elem(const uint16_t* p, size_t i) {
    return __builtin_bit_cast(float, (uint32_t)p[i] << 16);
}
__device__ __forceinline__ float load_elem(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ void store_elem(uint16_t* p, size_t i, float v) {
    p[i] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
}
__device__ __forceinline__ void store_elem(float* p, size_t i, float v) { p[i] = v; }

constexpr int kRowSlots = 4; // elements per lane (B <= 256)

// codes of v[0..3] for scale s (same arithmetic as quantize16)
__device__ __forceinline__ void quantize4(const float (&v)[kRowSlots], float s, int8_t (&q)[kRowSlots]) {
    if (s >= kFastQuotientMinScale) {
        const float r = 1.0f / s;
#pragma unroll
        for (int t = 0; t < kRowSlots; ++t) {
            float y = v[t] * r;
            const float e = __builtin_fmaf(-y, s, v[t]);
            y = __builtin_fmaf(e, r, y);
            q[t] = (int8_t)(code_bits_of(y) & 0xFFu);
        }
    } else if (s != 0.0f) {
#pragma unroll
        for (int t = 0; t < kRowSlots; ++t) q[t] = (int8_t)(code_bits_of(v[t] / s) & 0xFFu);
    } else {
#pragma unroll
        for (int t = 0; t < kRowSlots; ++t) q[t] = 0;
    }
}

__device__ __forceinline__ size_t wave_block_index() {
    return (size_t)blockIdx.x * (kThreads / 64) + threadIdx.x / 64;
}

template <typename In>
__global__ __launch_bounds__(kThreads) void k_quantize_rows(const In* __restrict__ x, RowMap map, size_t nblocks,
                                                            int8_t* __restrict__ codes, float* __restrict__ scales) {
    const size_t b = wave_block_index();
    if (b >= nblocks) return; // whole wavefronts leave together
    const int lane = threadIdx.x & 63;
    size_t start;
    uint32_t len;
    map.locate(b, start, len);
    float v[kRowSlots];
    float m = 0.0f;
#pragma unroll
    for (int t = 0; t < kRowSlots; ++t) {
        const uint32_t i = lane + 64 * t;
        v[t] = i < len ? load_elem(x, start + i) : 0.0f;
        m = fmaxf(m, fabsf(v[t]));
    }
    const float s = wave_max(m) / 127.0f;
    int8_t q[kRowSlots];
    quantize4(v, s, q);
#pragma unroll
    for (int t = 0; t < kRowSlots; ++t) {
        const uint32_t i = lane + 64 * t;
        if (i < len) codes[start + i] = q[t];
    }
    if (lane == 0) scales[b] = s;
}

template <typename Out>
__global__ __launch_bounds__(kThreads) void k_dequantize_rows(const int8_t* __restrict__ codes,
                                                              const float* __restrict__ scales, RowMap map,
                                                              size_t nblocks, Out* __restrict__ out) {
    const size_t b = wave_block_index();
    if (b >= nblocks) return;
    const int lane = threadIdx.x & 63;
    size_t start;
    uint32_t len;
    map.locate(b, start, len);
    const float s = scales[b];
#pragma unroll
    for (int t = 0; t < kRowSlots; ++t) {
        const uint32_t i = lane + 64 * t;
        if (i < len) store_elem(out, start + i, (float)codes[start + i] * s);
    }
}

template <typename Out>
__global__ __launch_bounds__(kThreads) void k_reduce_rows(RankPtrs rp, int nranks, RowMap map, size_t nblocks,
                                                          int8_t* codes_out, float* scales_out, Out* out) {
    const size_t b = wave_block_index();
    if (b >= nblocks) return;
    const int lane = threadIdx.x & 63;
    size_t start;
    uint32_t len;
    map.locate(b, start, len);
    float acc[kRowSlots];
    for (int r = 0; r < nranks; ++r) {
        const float s = rp.scales[r][b];
#pragma unroll
        for (int t = 0; t < kRowSlots; ++t) {
            const uint32_t i = lane + 64 * t;
            const float y = i < len ? (float)rp.codes[r][start + i] * s : 0.0f;
            acc[t] = r == 0 ? y : acc[t] + y;
        }
    }
    float m = 0.0f;
#pragma unroll
    for (int t = 0; t < kRowSlots; ++t) m = fmaxf(m, fabsf(acc[t]));
    const float so = wave_max(m) / 127.0f;
    int8_t q[kRowSlots];
    quantize4(acc, so, q);
    // every lane has read its inputs (the reduction above waited for them),
    // so writing in place over rank buffers is safe
#pragma unroll
    for (int t = 0; t < kRowSlots; ++t) {
        const uint32_t i = lane + 64 * t;
        if (i < len) {
            codes_out[start + i] = q[t];
            if (out) store_elem(out, start + i, (float)q[t] * so);
        }
    }
    if (lane == 0) scales_out[b] = so;
}

template <typename In>
__global__ __launch_bounds__(kThreads) void k_ring_step_rows(const int8_t* codes_in, const float* scales_in,
                                                             const In* __restrict__ local, RowMap map, size_t nblocks,
                                                             int8_t* codes_out, float* scales_out) {
    const size_t b = wave_block_index();
    if (b >= nblocks) return;
    const int lane = threadIdx.x & 63;
    size_t start;
    uint32_t len;
    map.locate(b, start, len);
    const float s = scales_in[b];
    float acc[kRowSlots];
    float m = 0.0f;
#pragma unroll
    for (int t = 0; t < kRowSlots; ++t) {
        const uint32_t i = lane + 64 * t;
        acc[t] = i < len ? (float)codes_in[start + i] * s + load_elem(local, start + i) : 0.0f;
        m = fmaxf(m, fabsf(acc[t]));
    }
    const float so = wave_max(m) / 127.0f;
    int8_t q[kRowSlots];
    quantize4(acc, so, q);
#pragma unroll
    for (int t = 0; t < kRowSlots; ++t) {
        const uint32_t i = lane + 64 * t;
        if (i < len) codes_out[start + i] = q[t];
    }
    if (lane == 0) scales_out[b] = so;
}

// ---------------------------------------------------------------------------
// launchers

namespace {

constexpr uint32_t kMaxGrid = 1u << 22;

struct Grid {
    uint32_t ntiles, blocks;
};

Grid grid_for(size_t n) {
    const size_t tiles = (n + kTileElems - 1) / kTileElems;
    Grid g;
    g.ntiles = (uint32_t)tiles;
    g.blocks = (uint32_t)(tiles < kMaxGrid ? tiles : kMaxGrid);
    return g;
}

template <int B>
hipError_t quantize_b(const void* x, int in_kind, size_t n, int8_t* codes, float* scales, hipStream_t st) {
    const Grid g = grid_for(n);
    if (in_kind == kInBF16)
        hipLaunchKernelGGL((k_quantize<B, uint16_t>), dim3(g.blocks), dim3(kThreads), 0, st,
                           static_cast<const uint16_t*>(x), n, codes, scales, g.ntiles);
    else
        hipLaunchKernelGGL((k_quantize<B, float>), dim3(g.blocks), dim3(kThreads), 0, st,
                           static_cast<const float*>(x), n, codes, scales, g.ntiles);
    return hipGetLastError();
}

template <int B>
hipError_t reduce_b(const RankPtrs& rp, int nranks, size_t n, int8_t* codes_out, float* scales_out,
                    void* out, int out_kind, hipStream_t st) {
    const Grid g = grid_for(n);
    if (out_kind == kOutBF16)
        hipLaunchKernelGGL((k_reduce<B, kOutBF16>), dim3(g.blocks), dim3(kThreads), 0, st, rp, nranks, n,
                           codes_out, scales_out, out, g.ntiles);
    else if (out_kind == kOutF32)
        hipLaunchKernelGGL((k_reduce<B, kOutF32>), dim3(g.blocks), dim3(kThreads), 0, st, rp, nranks, n,
                           codes_out, scales_out, out, g.ntiles);
    else
        hipLaunchKernelGGL((k_reduce<B, kOutNone>), dim3(g.blocks), dim3(kThreads), 0, st, rp, nranks, n,
                           codes_out, scales_out, out, g.ntiles);
    return hipGetLastError();
}

template <int B>
hipError_t ring_b(const int8_t* codes_in, const float* scales_in, const void* local, int in_kind,
                  size_t n, int8_t* codes_out, float* scales_out, hipStream_t st) {
    const Grid g = grid_for(n);
    if (in_kind == kInBF16)
        hipLaunchKernelGGL((k_ring_step<B, uint16_t>), dim3(g.blocks), dim3(kThreads), 0, st, codes_in,
                           scales_in, static_cast<const uint16_t*>(local), n, codes_out, scales_out,
                           g.ntiles);
    else
        hipLaunchKernelGGL((k_ring_step<B, float>), dim3(g.blocks), dim3(kThreads), 0, st, codes_in,
                           scales_in, static_cast<const float*>(local), n, codes_out, scales_out,
                           g.ntiles);
    return hipGetLastError();
}

template <int B>
hipError_t dequantize_b(const int8_t* codes, const float* scales, size_t n, void* out, int out_kind,
                        hipStream_t st) {
    const Grid g = grid_for(n);
    if (out_kind == kOutBF16)
        hipLaunchKernelGGL((k_dequantize<B, uint16_t>), dim3(g.blocks), dim3(kThreads), 0, st, codes,
                           scales, n, static_cast<uint16_t*>(out), g.ntiles);
    else
        hipLaunchKernelGGL((k_dequantize<B, float>), dim3(g.blocks), dim3(kThreads), 0, st, codes, scales,
                           n, static_cast<float*>(out), g.ntiles);
    return hipGetLastError();
}

uint32_t row_grid(size_t nblocks) { return (uint32_t)((nblocks + kThreads / 64 - 1) / (kThreads / 64)); }

} // namespace

hipError_t launch_rows(const RowsCall& c, hipStream_t st) {
    RowMap map;
    map.rows = c.rows;
    map.row_len = c.row_len;
    map.block = (uint32_t)c.block;
    map.per_row = (uint32_t)((c.row_len + c.block - 1) / c.block);
    const size_t nblocks = c.rows * map.per_row;
    const dim3 grid(row_grid(nblocks)), threads(kThreads);
    switch (c.op) {
    case kRowsQuantize:
        if (c.kind == kInBF16)
            hipLaunchKernelGGL((k_quantize_rows<uint16_t>), grid, threads, 0, st, static_cast<const uint16_t*>(c.x),
                               map, nblocks, c.codes_out, c.scales_out);
        else
            hipLaunchKernelGGL((k_quantize_rows<float>), grid, threads, 0, st, static_cast<const float*>(c.x), map,
                               nblocks, c.codes_out, c.scales_out);
        break;
    case kRowsDequantize:
        if (c.kind == kInBF16)
            hipLaunchKernelGGL((k_dequantize_rows<uint16_t>), grid, threads, 0, st, c.codes_in, c.scales_in, map,
                               nblocks, static_cast<uint16_t*>(c.out));
        else
            hipLaunchKernelGGL((k_dequantize_rows<float>), grid, threads, 0, st, c.codes_in, c.scales_in, map,
                               nblocks, static_cast<float*>(c.out));
        break;
    case kRowsReduce:
        if (c.kind == kInBF16)
            hipLaunchKernelGGL((k_reduce_rows<uint16_t>), grid, threads, 0, st, c.rp, c.nranks, map, nblocks,
                               c.codes_out, c.scales_out, static_cast<uint16_t*>(c.out));
        else
            hipLaunchKernelGGL((k_reduce_rows<float>), grid, threads, 0, st, c.rp, c.nranks, map, nblocks,
                               c.codes_out, c.scales_out, static_cast<float*>(c.out));
        break;
    default:
        if (c.kind == kInBF16)
            hipLaunchKernelGGL((k_ring_step_rows<uint16_t>), grid, threads, 0, st, c.codes_in, c.scales_in,
                               static_cast<const uint16_t*>(c.x), map, nblocks, c.codes_out, c.scales_out);
        else
            hipLaunchKernelGGL((k_ring_step_rows<float>), grid, threads, 0, st, c.codes_in, c.scales_in,
                               static_cast<const float*>(c.x), map, nblocks, c.codes_out, c.scales_out);
        break;
    }
    return hipGetLastError();
}

hipError_t launch_reduce_unquantized(const PlainPtrs& xp, int nranks, size_t n, int kind, void* out,
                                     hipStream_t st) {
    const Grid g = grid_for(n);
    if (kind == kInBF16)
        hipLaunchKernelGGL((k_reduce_unquantized<uint16_t>), dim3(g.blocks), dim3(kThreads), 0, st, xp, nranks, n,
                           static_cast<uint16_t*>(out), g.ntiles);
    else
        hipLaunchKernelGGL((k_reduce_unquantized<float>), dim3(g.blocks), dim3(kThreads), 0, st, xp, nranks, n,
                           static_cast<float*>(out), g.ntiles);
    return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int in_kind, size_t n, int block, int8_t* codes, float* scales,
                           hipStream_t st) {
    switch (block) {
    case 64: return quantize_b<64>(x, in_kind, n, codes, scales, st);
    case 128: return quantize_b<128>(x, in_kind, n, codes, scales, st);
    default: return quantize_b<256>(x, in_kind, n, codes, scales, st);
    }
}

hipError_t launch_reduce(const RankPtrs& rp, int nranks, size_t n, int block, int8_t* codes_out,
                         float* scales_out, void* out, int out_kind, hipStream_t st) {
    switch (block) {
    case 64: return reduce_b<64>(rp, nranks, n, codes_out, scales_out, out, out_kind, st);
    case 128: return reduce_b<128>(rp, nranks, n, codes_out, scales_out, out, out_kind, st);
    default: return reduce_b<256>(rp, nranks, n, codes_out, scales_out, out, out_kind, st);
    }
}

hipError_t launch_ring_step(const int8_t* codes_in, const float* scales_in, const void* local, int in_kind,
                            size_t n, int block, int8_t* codes_out, float* scales_out, hipStream_t st) {
    switch (block) {
    case 64: return ring_b<64>(codes_in, scales_in, local, in_kind, n, codes_out, scales_out, st);
    case 128: return ring_b<128>(codes_in, scales_in, local, in_kind, n, codes_out, scales_out, st);
    default: return ring_b<256>(codes_in, scales_in, local, in_kind, n, codes_out, scales_out, st);
    }
}

hipError_t launch_dequantize(const int8_t* codes, const float* scales, size_t n, int block, void* out,
                             int out_kind, hipStream_t st) {
    switch (block) {
    case 64: return dequantize_b<64>(codes, scales, n, out, out_kind, st);
    case 128: return dequantize_b<128>(codes, scales, n, out, out_kind, st);
    default: return dequantize_b<256>(codes, scales, n, out, out_kind, st);
    }
}

} // namespace qar
