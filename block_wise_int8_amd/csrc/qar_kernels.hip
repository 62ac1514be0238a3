// qar_kernels.hip -- libqar's gfx950 kernels and their launchers.
//
// Method: EQuARX ("EQuARX: Efficient Quantized AllReduce in XLA for
// Distributed Machine Learning Acceleration"), page summary, section
// "technical framework": blocks (step 1), dynamic per-block quantization to
// INT8 (step 2, with the run-time range of "key design" item 1), reduction of
// quantized contributions (step 3), dequantization (step 4).  The flat kernels
// take the code format as a policy: Int8Codes; E4M3Codes for the FP8 variant
// of the TACO page, section 2.A "Waarom FP8?" (one byte per element as
// well); Int4Codes, the int8 rules at 4 bits with two codes per byte.  The
// arithmetic each kernel performs is spelled out in include/qar.h.
//
// Every kernel streams HBM once: 16-byte loads and stores per lane (8-byte
// code accesses for 4-bit codes), a block's absmax by DPP inside its lanes,
// the requantization fused behind the reduction so the fp32 sum never leaves
// registers.  A workgroup walks tiles
// of 4096 elements with a grid-stride loop (the grid is capped, the loop
// covers any n).
#include <mutex>
#include <tuple>
#include <type_traits>
#include <utility>

#include "qar_device.h"
#include "qar_launch.h"

namespace qar {

// ---------------------------------------------------------------------------
// where each lane works
//
// Global lane g owns P consecutive elements starting at e0, inside block
// blk; the B/P lanes of a block are adjacent (one DPP row, part of one, or
// two).  P is 16 (FlatLanes, RowLanes) or 8 (FlatLanes8, RowLanes8: the
// reduce's narrow kernels).
//   Flat: blocks tile the buffer: e0 = P g, blk = e0 / B.
//   Rows: row-bounded blocks of a [rows, row_len] tensor with
//         row_len % 16 == 0: block blk = (row r, k-th block of the row)
//         starts at r * row_len + k * B; lanes past the end of a row's
//         partial last block are invalid and contribute nothing to the
//         block's absmax.
// Invalid lanes read element 0 (any finite value) and store nothing.
struct LaneAt {
    size_t e0, blk;
    bool valid, leads; // leads: first lane of its block (writes the scale)
};

constexpr int kLaneElems8 = 8;

template <int B, int P>
__device__ __forceinline__ LaneAt flat_lane(size_t g, size_t n) {
    LaneAt a;
    a.e0 = g * P;
    a.valid = a.e0 < n;
    a.blk = a.e0 / B;
    a.leads = a.e0 % B == 0;
    return a;
}

template <int B, int P>
__device__ __forceinline__ LaneAt row_lane(size_t g, size_t row_len, size_t nblocks, uint32_t per_row) {
    constexpr uint32_t L = B / P;
    LaneAt a;
    a.blk = g / L;
    const uint32_t j = (uint32_t)(g % L);
    const uint32_t b32 = (uint32_t)a.blk; // nblocks < 2^26
    const uint32_t r = b32 / per_row, k = b32 - r * per_row;
    const size_t col = (size_t)k * B + (size_t)j * P;
    a.e0 = (size_t)r * row_len + col;
    a.valid = a.blk < nblocks && col < row_len;
    a.leads = j == 0;
    return a;
}

template <int B>
struct FlatLanes {
    size_t n;
    static constexpr int kLane = kLaneElems;
    static constexpr bool kContiguous = true; // a wave covers 1024 consecutive elements
    static constexpr bool kPartialBlocks = false;
    __device__ __forceinline__ LaneAt at(size_t g) const { return flat_lane<B, kLane>(g, n); }
};

template <int B>
struct RowLanes {
    size_t row_len, nblocks;
    uint32_t per_row; // blocks per row
    static constexpr int kLane = kLaneElems;
    static constexpr bool kContiguous = false;
    static constexpr bool kPartialBlocks = true;
    __device__ __forceinline__ LaneAt at(size_t g) const { return row_lane<B, kLane>(g, row_len, nblocks, per_row); }
};

template <int B>
struct FlatLanes8 {
    size_t n;
    static constexpr int kLane = kLaneElems8;
    static constexpr bool kContiguous = true; // a wave covers 512 consecutive elements
    static constexpr bool kPartialBlocks = false;
    __device__ __forceinline__ LaneAt at(size_t g) const { return flat_lane<B, kLane>(g, n); }
};

template <int B>
struct RowLanes8 {
    size_t row_len, nblocks;
    uint32_t per_row;
    static constexpr int kLane = kLaneElems8;
    static constexpr bool kContiguous = false;
    static constexpr bool kPartialBlocks = true;
    __device__ __forceinline__ LaneAt at(size_t g) const { return row_lane<B, kLane>(g, row_len, nblocks, per_row); }
};

// absmax over a lane's values, zero for an invalid lane of a partial block
template <typename Lanes>
__device__ __forceinline__ float masked_absmax(const float (&v)[kLaneElems], bool valid) {
    const float m = lane_absmax(v);
    if constexpr (Lanes::kPartialBlocks) return valid ? m : 0.0f;
    return m;
}

// ---------------------------------------------------------------------------
// quantize: x (bf16 or fp32) -> codes, scales

template <int B, typename In, typename Lanes, typename C = Int8Codes>
__global__ __launch_bounds__(kThreads) void k_quantize(const In* __restrict__ x, Lanes lanes,
                                                       int8_t* __restrict__ codes,
                                                       float* __restrict__ scales,
                                                       uint32_t ntiles) {
    for (uint32_t tile = xcd_tile(blockIdx.x, gridDim.x); tile < ntiles; tile += gridDim.x) {
        const LaneAt a = lanes.at((size_t)tile * kThreads + threadIdx.x);
        const size_t ld = a.valid ? a.e0 : 0;
        float v[kLaneElems];
        load16(x + ld, v);
        const float s = block_max<B>(masked_absmax<Lanes>(v, a.valid)) / C::kQmax;
        const typename C::Vec q = C::quantize(v, s);
        if (a.valid) {
            C::store(codes, a.e0, q);
            if (a.leads) scales[a.blk] = s;
        }
    }
}

// ---------------------------------------------------------------------------
// slot layout: flat kernels that stream bf16/fp32 data
//
// Above, a lane owns 16 consecutive elements, which keeps its 16 codes in
// one 16-byte vector but spreads a wavefront's data loads: 2 (bf16) or 4
// (fp32) loads per lane, each covering only part of every 32- or 64-byte
// stretch it touches.  For the flat quantize and ring step a lane instead
// owns 16-byte slots of the data: with P = 16 / sizeof(element) (8 for
// bf16, 4 for fp32), lane L of a wavefront owns elements P*L + 64*P*j ..
// + P-1 (j = 0 .. 16/P - 1) of the wave's 1024-element tile.  Every data
// load then covers 1 KB of contiguous memory, and the P codes of a slot
// (P or P/2 bytes) lie contiguous across the wave as well.  A block of B
// elements is B/P adjacent lanes of one slot (8 to 64 lanes).  Measured on
// the fp32 quantize of 67M elements: 82.0 -> 56.6 us, and HBM reads from
// 1.085 to 1.00 times the input bytes.  bf16 data (32 bytes per lane in the
// layout above) measured slightly slower in slots (quantize of 16.8M
// elements 11.1 against 10.6 us, the ring step 7.6 against 7.5 us), so the
// launchers give the slot kernels fp32 data only.

__device__ __forceinline__ void unpack_slot(uint4 r, float (&v)[8]) { // 8 bf16
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[2 * k] = bf16_lo(w[k]);
        v[2 * k + 1] = bf16_hi(w[k]);
    }
}

__device__ __forceinline__ void unpack_slot(uint4 r, float (&v)[4]) { // 4 fp32
    v[0] = __builtin_bit_cast(float, r.x);
    v[1] = __builtin_bit_cast(float, r.y);
    v[2] = __builtin_bit_cast(float, r.z);
    v[3] = __builtin_bit_cast(float, r.w);
}

template <typename In>
struct SlotShape {
    static constexpr int P = 16 / (int)sizeof(In); // elements per slot
    static constexpr int J = kLaneElems / P;       // slots per lane
    // element of slot j of this lane, in the wave tile that starts at wave0
    static __device__ __forceinline__ size_t at(size_t wave0, int j, int lane) {
        return wave0 + (size_t)(64 * P * j + P * lane);
    }
};

__device__ __forceinline__ size_t wave_tile_start(uint32_t tile) {
    return ((size_t)tile * kThreads + (threadIdx.x & ~63u)) * kLaneElems;
}

template <int B, typename In, typename C = Int8Codes>
__global__ __launch_bounds__(kThreads) void k_quantize_slots(const In* __restrict__ x, size_t n,
                                                             int8_t* __restrict__ codes, float* __restrict__ scales,
                                                             uint32_t ntiles) {
    using S = SlotShape<In>;
    constexpr int P = S::P, L = B / P;
    const int lane = threadIdx.x & 63;
    for (uint32_t tile = xcd_tile(blockIdx.x, gridDim.x); tile < ntiles; tile += gridDim.x) {
        const size_t wave0 = wave_tile_start(tile);
        uint4 raw[S::J];
#pragma unroll
        for (int j = 0; j < S::J; ++j) {
            const size_t e = S::at(wave0, j, lane);
            raw[j] = load_b128(x + (e < n ? e : 0)); // n % B == 0: a block is wholly inside or outside
        }
#pragma unroll
        for (int j = 0; j < S::J; ++j) {
            const size_t e = S::at(wave0, j, lane);
            float v[P];
            unpack_slot(raw[j], v);
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < P; ++i) m = fmaxf(m, fabsf(v[i]));
            const float s = lanes_max<L>(m) / C::kQmax;
            const auto q = C::template quantize_p<P>(v, s);
            if (e < n) {
                C::template store_p<P>(codes, e, q);
                if (e % B == 0) scales[e / B] = s;
            }
        }
    }
}

// ring step in the slot layout; codes_out / scales_out may be codes_in /
// scales_in (every lane reads its own codes and its blocks' scales before it
// writes them)
template <int B, typename In, typename C = Int8Codes>
__global__ __launch_bounds__(kThreads) void k_ring_step_slots(const int8_t* codes_in, const float* scales_in,
                                                              const In* __restrict__ local, size_t n,
                                                              int8_t* codes_out, float* scales_out, uint32_t ntiles) {
    using S = SlotShape<In>;
    constexpr int P = S::P, L = B / P;
    using Pack = typename C::template Pack<P>;
    const int lane = threadIdx.x & 63;
    for (uint32_t tile = xcd_tile(blockIdx.x, gridDim.x); tile < ntiles; tile += gridDim.x) {
        const size_t wave0 = wave_tile_start(tile);
        uint4 raw[S::J];
        Pack q[S::J];
        float s[S::J];
#pragma unroll
        for (int j = 0; j < S::J; ++j) {
            const size_t e = S::at(wave0, j, lane);
            const size_t ld = e < n ? e : 0;
            raw[j] = load_b128(local + ld);
            q[j] = C::template load_p<P>(codes_in, ld);
            s[j] = scales_in[ld / B];
        }
#pragma unroll
        for (int j = 0; j < S::J; ++j) {
            const size_t e = S::at(wave0, j, lane);
            float acc[P], x[P];
            C::template dequantize_p<P>(q[j], s[j], acc);
            unpack_slot(raw[j], x);
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < P; ++i) {
                acc[i] = acc[i] + x[i];
                m = fmaxf(m, fabsf(acc[i]));
            }
            const float so = lanes_max<L>(m) / C::kQmax;
            const Pack qo = C::template quantize_p<P>(acc, so);
            if (e < n) {
                C::template store_p<P>(codes_out, e, qo);
                if (e % B == 0) scales_out[e / B] = so;
            }
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
template <int B, int OUT, typename C = Int8Codes>
__device__ __forceinline__ void store_dequantized_tile(typename C::Vec qo, float so, size_t e0, size_t n, void* out,
                                                       typename C::Vec* lds_codes, float* lds_scales) {
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
            float y[8];
            C::scaled8(codes, e, lds_scales[e / B], y);
            uint4 o;
            o.x = pack_bf16x2(y[0], y[1]);
            o.y = pack_bf16x2(y[2], y[3]);
            o.z = pack_bf16x2(y[4], y[5]);
            o.w = pack_bf16x2(y[6], y[7]);
            if (wave0 + e < n) store_b128(static_cast<uint16_t*>(out) + wave0 + e, o);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 256 * j + 4 * lane;
            float y[4];
            C::scaled4(codes, e, lds_scales[e / B], y);
            uint4 o;
            o.x = __builtin_bit_cast(uint32_t, y[0]);
            o.y = __builtin_bit_cast(uint32_t, y[1]);
            o.z = __builtin_bit_cast(uint32_t, y[2]);
            o.w = __builtin_bit_cast(uint32_t, y[3]);
            if (wave0 + e < n) store_b128(static_cast<float*>(out) + wave0 + e, o);
        }
    }
    // the next tile overwrites the staging area: keep this tile's reads first
    __builtin_amdgcn_wave_barrier();
}

// A line of zeros that the reduce reads in place of a rank slot it does not
// use (past the last rank, or rank own, whose codes are made in registers),
// so that every slot of a group is loaded without a branch.  Never written.
__device__ __align__(64) uint32_t g_unused_slot[16];

// The reduce over the tiles of one workgroup.  With OwnIn not void, rank
// `own` is quantized from x_own in the same pass: its codes and scale are
// written for the peers and the same register values enter the sum, so the
// result equals a quantize followed by the plain reduce.
//
// kDense: every slot of a load group is loaded, an unused one (rank own,
// whose codes are made in registers, or past the last rank) reading
// g_unused_slot, which lets the compiler wait for each rank's data on its own
// instead of for the whole group.  Measured on the step (own rank, N ranks):
// 3-5% faster for N = 5..8 and 16, but each slot past the last rank costs a
// load, so with 1-4 ranks in the last group (N = 2: 16% slower) the loads
// branch around the unused slots instead; the launcher picks by N.  The
// plain reduce always branches (the dense form measured 4% slower there).
//
// G ranks' loads are in flight together, one group after another.  The
// plain reduce without output takes G = 16 from 9 ranks on (N = 16 × 67M,
// B = 64: 207.9 -> 199.3 µs as one launch, 203.2 -> 199.1 µs in 8 chunks
// over 4 streams; 124 VGPRs instead of 78, still 4 waves per SIMD).  With a
// fused output G = 16 needs 131-142 VGPRs and the step 157 (3 waves per
// SIMD); on 16.8M bf16, B = 256, with bf16 output (µs, G = 8 -> 16): reduce
// N = 16 54.8 -> 54.5, N = 32 102.4 -> 104.9; step N = 16 59.9 -> 59.7,
// N = 32 109.0 -> 110.0.  So those keep 8.
template <int B, int OUT, typename Lanes, typename OwnIn, typename C, bool kDense = false, int G = 8>
__device__ __forceinline__ void reduce_tiles(RankPtrs rp, int nranks, Lanes lanes, int8_t* codes_out,
                                             float* scales_out, void* __restrict__ out, uint32_t ntiles,
                                             const OwnIn* __restrict__ x_own, int own,
                                             int8_t* __restrict__ own_codes, float* __restrict__ own_scales,
                                             TileMap map) {
    constexpr bool kOwn = !std::is_void<OwnIn>::value;
    constexpr bool kStaged = OUT != kOutNone && Lanes::kContiguous;
    using Vec = typename C::Vec;
    __shared__ Vec lds_codes[kStaged ? kThreads : 1];
    __shared__ float lds_scales[kStaged ? kThreads * kLaneElems / B : 1];
    for (uint32_t t = map.first(blockIdx.x, gridDim.x); t < ntiles; t += gridDim.x) {
        const uint32_t tile = map.tile(t);
        const LaneAt a = lanes.at((size_t)tile * kThreads + threadIdx.x);
        const size_t ld = a.valid ? a.e0 : 0;
        const size_t blk = a.valid ? a.blk : 0;
        // rank own's raw data is loaded first and converted while the first
        // group's codes are in flight
        using OwnRaw = Raw16<std::conditional_t<kOwn, OwnIn, uint16_t>>;
        OwnRaw xr{};
        if constexpr (kOwn) xr = load_raw16(x_own + ld);
        Vec q_own{};
        float s_own = 0.0f;
        float acc[kLaneElems];
        for (int g = 0; g < nranks; g += G) {
            Vec q[G];
            float s[G];
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const bool used = g + j < nranks && !(kOwn && g + j == own);
                if constexpr (kDense) {
                    const int8_t* c = used ? rp.codes[g + j] : reinterpret_cast<const int8_t*>(g_unused_slot);
                    const float* sc = used ? rp.scales[g + j] : reinterpret_cast<const float*>(g_unused_slot);
                    q[j] = C::load(c, used ? ld : 0);
                    s[j] = sc[used ? blk : 0];
                } else if (used) {
                    q[j] = C::load(rp.codes[g + j], ld);
                    s[j] = rp.scales[g + j][blk];
                }
            }
            if constexpr (kOwn) {
                if (g == 0) {
                    float v[kLaneElems];
                    unpack16(xr, v);
                    s_own = block_max<B>(masked_absmax<Lanes>(v, a.valid)) / C::kQmax;
                    q_own = C::quantize(v, s_own);
                    if (a.valid) {
                        C::store(own_codes, a.e0, q_own);
                        if (a.leads) own_scales[a.blk] = s_own;
                    }
                }
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    if (g + j == own) {
                        q[j] = q_own;
                        s[j] = s_own;
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < G; ++j) {
                if (g + j < nranks) {
                    float y[kLaneElems];
                    C::dequantize(q[j], s[j], y);
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
        const float so = block_max<B>(masked_absmax<Lanes>(acc, a.valid)) / C::kQmax;
        uint32_t w[kLaneElems];
        Vec qo;
        if constexpr (OUT != kOutNone && !kStaged) {
            static_assert(std::is_same<C, Int8Codes>::value, "row-bounded output is int8 only");
            qo = quantize16(acc, so, w);
        } else {
            qo = C::quantize(acc, so);
        }
        if (a.valid) {
            C::store(codes_out, a.e0, qo);
            if (a.leads) scales_out[a.blk] = so;
        }
        if constexpr (kStaged) {
            const int wave = threadIdx.x / 64;
            store_dequantized_tile<B, OUT, C>(qo, so, a.e0, lanes.n, out, lds_codes + wave * 64,
                                           lds_scales + wave * (64 * kLaneElems / B));
        } else if constexpr (OUT != kOutNone) {
            // row-bounded blocks: a wave's elements are not one contiguous
            // range, so each lane stores its own 16 values
            if (a.valid) {
                float y[kLaneElems];
                dequantize_words(w, so, y);
                if constexpr (OUT == kOutBF16)
                    store16(static_cast<uint16_t*>(out) + a.e0, y);
                else
                    store16(static_cast<float*>(out) + a.e0, y);
            }
        }
    }
}

template <int B, int OUT, typename Lanes, typename C = Int8Codes, int G = 8>
__global__ __launch_bounds__(kThreads) void k_reduce(RankPtrs rp, int nranks, Lanes lanes,
                                                     int8_t* codes_out, float* scales_out,
                                                     void* __restrict__ out, uint32_t ntiles, TileMap map) {
    reduce_tiles<B, OUT, Lanes, void, C, false, G>(rp, nranks, lanes, codes_out, scales_out, out, ntiles, nullptr,
                                                   -1, nullptr, nullptr, map);
}

template <int B, int OUT, typename In, typename C = Int8Codes, bool kDense = true>
__global__ __launch_bounds__(kThreads) void k_quantize_reduce(const In* __restrict__ x_own, int own,
                                                              int8_t* own_codes, float* own_scales,
                                                              RankPtrs rp, int nranks, FlatLanes<B> lanes,
                                                              int8_t* codes_out, float* scales_out,
                                                              void* __restrict__ out, uint32_t ntiles, uint32_t super) {
    reduce_tiles<B, OUT, FlatLanes<B>, In, C, kDense>(rp, nranks, lanes, codes_out, scales_out, out, ntiles, x_own,
                                                      own, own_codes, own_scales, TileMap{super, 0, 1, 1});
}

// ---------------------------------------------------------------------------
// the same reduce and one-kernel step with 8 elements per lane
//
// A workgroup of 256 lanes takes 2048 elements, so a given n launches twice
// the wavefronts, each with half the registers and half the arithmetic after
// its last load.  A lane's 8 codes are 8 bytes (4 for 4-bit codes),
// contiguous across the wavefront, and so are its 8 bf16 inputs and outputs
// (16 bytes), so a bf16 output needs no staging (an fp32 output goes
// through store_f32_tile8).  A block of B elements is B/8 adjacent lanes (8
// to 32) of one wavefront.  Lanes is FlatLanes8 or, for the row-bounded
// reduce, RowLanes8.  The launchers below say where these kernels are used
// and what was measured.
constexpr int kTileElems8 = kThreads * kLaneElems8;

// The fp32 output of a wave's 512 elements with 8 elements per lane: a
// lane's 8 results are 32 bytes, so two direct 16-byte stores per lane each
// cover alternate halves of every 32 bytes (counters: 6.7% more bytes
// written than the output's size).  As store_dequantized_tile does for 16
// per lane, the wave puts its codes and block scales in LDS, and each lane
// dequantizes the 4 codes of the 16-byte slots at wave elements 4 lane +
// 256 j (j = 0, 1), so that each store instruction writes whole lines.  A
// slot's destination is that of the lane that holds it (lane 32 j + lane/2,
// its half lane & 1): for flat lanes the wave's elements are consecutive;
// for row-bounded lanes each lane's start (or kNoSlot, invalid) goes
// through LDS as well.
constexpr size_t kNoSlot = ~(size_t)0;

template <int B, typename C, bool kContiguous>
__device__ __forceinline__ void store_f32_tile8(typename C::template Pack<kLaneElems8> qo, float so, size_t e0,
                                                bool valid, size_t n, float* out,
                                                typename C::template Pack<kLaneElems8>* lds_codes,
                                                float* lds_scales, size_t* lds_e0) {
    constexpr int kLanesPerBlock = B / kLaneElems8;
    const int lane = threadIdx.x & 63;
    lds_codes[lane] = qo;
    if (lane % kLanesPerBlock == 0) lds_scales[lane / kLanesPerBlock] = so;
    if constexpr (!kContiguous) lds_e0[lane] = valid ? e0 : kNoSlot;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int8_t* codes = reinterpret_cast<const int8_t*>(lds_codes);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = 256 * j + 4 * lane; // element of the wave's 512
        size_t dst;
        bool ok;
        if constexpr (kContiguous) {
            dst = e0 - (size_t)lane * kLaneElems8 + e;
            ok = dst < n;
        } else {
            const size_t start = lds_e0[e / kLaneElems8];
            ok = start != kNoSlot;
            dst = start + e % kLaneElems8;
        }
        float y[4];
        C::scaled4(codes, e, lds_scales[e / B], y);
        if (ok)
            store_b128(out + dst, make_uint4(__builtin_bit_cast(uint32_t, y[0]), __builtin_bit_cast(uint32_t, y[1]),
                                             __builtin_bit_cast(uint32_t, y[2]), __builtin_bit_cast(uint32_t, y[3])));
    }
    // the next tile overwrites the staging area: keep this tile's reads first
    __builtin_amdgcn_wave_barrier();
}

template <int B, int OUT, typename OwnIn, typename C, bool kDense, typename Lanes>
__device__ __forceinline__ void reduce_tiles8(RankPtrs rp, int nranks, Lanes lanes, int8_t* codes_out,
                                              float* scales_out, void* __restrict__ out, uint32_t ntiles,
                                              const OwnIn* __restrict__ x_own, int own,
                                              int8_t* __restrict__ own_codes, float* __restrict__ own_scales,
                                              TileMap map) {
    constexpr int G = 8; // ranks whose loads are in flight together
    constexpr int P = kLaneElems8, L = B / P;
    constexpr bool kOwn = !std::is_void<OwnIn>::value;
    using In = std::conditional_t<kOwn, OwnIn, uint16_t>;
    constexpr int kRawWords = P * (int)sizeof(In) / 16; // 16-byte words of own input per lane
    using Pack = typename C::template Pack<P>;
    constexpr bool kStaged = OUT == kOutF32;
    __shared__ Pack lds_codes[kStaged ? kThreads : 1];
    __shared__ float lds_scales[kStaged ? kThreads * P / B : 1];
    __shared__ size_t lds_e0[kStaged && !Lanes::kContiguous ? kThreads : 1];
    for (uint32_t t = map.first(blockIdx.x, gridDim.x); t < ntiles; t += gridDim.x) {
        const uint32_t tile = map.tile(t);
        const LaneAt a = lanes.at((size_t)tile * kThreads + threadIdx.x);
        const size_t ld = a.valid ? a.e0 : 0;
        const size_t blk = a.valid ? a.blk : 0;
        uint4 xr[kRawWords];
        if constexpr (kOwn) {
#pragma unroll
            for (int k = 0; k < kRawWords; ++k) xr[k] = load_b128(x_own + ld + k * (16 / sizeof(In)));
        }
        Pack q_own{};
        float s_own = 0.0f;
        float acc[P];
        for (int g = 0; g < nranks; g += G) {
            Pack q[G];
            float s[G];
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const bool used = g + j < nranks && !(kOwn && g + j == own);
                if constexpr (kDense) {
                    const int8_t* c = used ? rp.codes[g + j] : reinterpret_cast<const int8_t*>(g_unused_slot);
                    const float* sc = used ? rp.scales[g + j] : reinterpret_cast<const float*>(g_unused_slot);
                    q[j] = C::template load_p<P>(c, used ? ld : 0);
                    s[j] = sc[used ? blk : 0];
                } else if (used) {
                    q[j] = C::template load_p<P>(rp.codes[g + j], ld);
                    s[j] = rp.scales[g + j][blk];
                }
            }
            if constexpr (kOwn) {
                if (g == 0) {
                    float v[P];
                    if constexpr (std::is_same<In, float>::value) {
                        float lo[4], hi[4];
                        unpack_slot(xr[0], lo);
                        unpack_slot(xr[1], hi);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            v[i] = lo[i];
                            v[4 + i] = hi[i];
                        }
                    } else {
                        unpack_slot(xr[0], v);
                    }
                    float m = 0.0f;
#pragma unroll
                    for (int i = 0; i < P; ++i) m = fmaxf(m, fabsf(v[i]));
                    if constexpr (Lanes::kPartialBlocks) m = a.valid ? m : 0.0f;
                    s_own = lanes_max<L>(m) / C::kQmax;
                    q_own = C::template quantize_p<P>(v, s_own);
                    if (a.valid) {
                        C::template store_p<P>(own_codes, a.e0, q_own);
                        if (a.leads) own_scales[a.blk] = s_own;
                    }
                }
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    if (g + j == own) {
                        q[j] = q_own;
                        s[j] = s_own;
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < G; ++j) {
                if (g + j < nranks) {
                    float y[P];
                    C::template dequantize_p<P>(q[j], s[j], y);
                    if (g + j == 0) {
#pragma unroll
                        for (int i = 0; i < P; ++i) acc[i] = y[i];
                    } else {
#pragma unroll
                        for (int i = 0; i < P; ++i) acc[i] = acc[i] + y[i];
                    }
                }
            }
        }
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < P; ++i) m = fmaxf(m, fabsf(acc[i]));
        if constexpr (Lanes::kPartialBlocks) m = a.valid ? m : 0.0f;
        const float so = lanes_max<L>(m) / C::kQmax;
        const Pack qo = C::template quantize_p<P>(acc, so);
        if (a.valid) {
            const size_t e0 = a.e0;
            C::template store_p<P>(codes_out, e0, qo);
            if (a.leads) scales_out[a.blk] = so;
            if constexpr (OUT != kOutNone && !kStaged) {
                float y[P];
                C::template dequantize_p<P>(qo, so, y);
                if constexpr (OUT == kOutBF16) {
                    store_b128(static_cast<uint16_t*>(out) + e0,
                               make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                                          pack_bf16x2(y[6], y[7])));
                } else {
#pragma unroll
                    for (int k = 0; k < 2; ++k)
                        store_b128(static_cast<float*>(out) + e0 + 4 * k,
                                   make_uint4(__builtin_bit_cast(uint32_t, y[4 * k]),
                                              __builtin_bit_cast(uint32_t, y[4 * k + 1]),
                                              __builtin_bit_cast(uint32_t, y[4 * k + 2]),
                                              __builtin_bit_cast(uint32_t, y[4 * k + 3])));
                }
            }
        }
        if constexpr (kStaged) {
            const int wave = threadIdx.x / 64;
            size_t n = 0; // bounds the flat lanes' slots; row-bounded slots carry their own
            if constexpr (Lanes::kContiguous) n = lanes.n;
            store_f32_tile8<B, C, Lanes::kContiguous>(qo, so, a.e0, a.valid, n, static_cast<float*>(out),
                                                      lds_codes + wave * 64, lds_scales + wave * (64 * P / B),
                                                      lds_e0 + (Lanes::kContiguous ? 0 : wave * 64));
        }
    }
}

template <int B, int OUT, typename C>
__global__ __launch_bounds__(kThreads) void k_reduce8(RankPtrs rp, int nranks, size_t n, int8_t* codes_out,
                                                      float* scales_out, void* __restrict__ out, uint32_t ntiles,
                                                      TileMap map) {
    reduce_tiles8<B, OUT, void, C, false>(rp, nranks, FlatLanes8<B>{n}, codes_out, scales_out, out, ntiles,
                                          nullptr, -1, nullptr, nullptr, map);
}

// the row-bounded reduce (int8 codes) with 8 elements per lane
template <int B, int OUT>
__global__ __launch_bounds__(kThreads) void k_reduce8_rows(RankPtrs rp, int nranks, RowLanes8<B> lanes,
                                                           int8_t* codes_out, float* scales_out,
                                                           void* __restrict__ out, uint32_t ntiles) {
    reduce_tiles8<B, OUT, void, Int8Codes, false>(rp, nranks, lanes, codes_out, scales_out, out, ntiles, nullptr,
                                                  -1, nullptr, nullptr, TileMap{0, 0, 1, 1});
}

template <int B, int OUT, typename In, typename C, bool kDense>
__global__ __launch_bounds__(kThreads) void k_quantize_reduce8(const In* __restrict__ x_own, int own,
                                                               int8_t* own_codes, float* own_scales, RankPtrs rp,
                                                               int nranks, size_t n, int8_t* codes_out,
                                                               float* scales_out, void* __restrict__ out,
                                                               uint32_t ntiles, uint32_t super) {
    reduce_tiles8<B, OUT, In, C, kDense>(rp, nranks, FlatLanes8<B>{n}, codes_out, scales_out, out, ntiles, x_own,
                                         own, own_codes, own_scales, TileMap{super, 0, 1, 1});
}

// ---------------------------------------------------------------------------
// ring step: dequantize incoming + add local (bf16/fp32) + requantize

template <int B, typename In, typename Lanes, typename C = Int8Codes>
__global__ __launch_bounds__(kThreads) void k_ring_step(const int8_t* codes_in, const float* scales_in,
                                                        const In* __restrict__ local, Lanes lanes,
                                                        int8_t* codes_out, float* scales_out,
                                                        uint32_t ntiles) {
    for (uint32_t tile = xcd_tile(blockIdx.x, gridDim.x); tile < ntiles; tile += gridDim.x) {
        const LaneAt a = lanes.at((size_t)tile * kThreads + threadIdx.x);
        const size_t ld = a.valid ? a.e0 : 0;
        const size_t blk = a.valid ? a.blk : 0;
        float acc[kLaneElems];
        {
            const typename C::Vec q = C::load(codes_in, ld);
            const float s = scales_in[blk];
            float x[kLaneElems];
            load16(local + ld, x);
            C::dequantize(q, s, acc);
#pragma unroll
            for (int i = 0; i < kLaneElems; ++i) acc[i] = acc[i] + x[i];
        }
        const float so = block_max<B>(masked_absmax<Lanes>(acc, a.valid)) / C::kQmax;
        const typename C::Vec qo = C::quantize(acc, so);
        if (a.valid) {
            C::store(codes_out, a.e0, qo);
            if (a.leads) scales_out[a.blk] = so;
        }
    }
}

// ---------------------------------------------------------------------------
// dequantize: codes, scales -> bf16 or fp32

// Each 16-byte store instruction writes 1 KB of contiguous output: lane L of
// a wavefront owns the store slots at elements 8L + 512j (bf16, j = 0..1) or
// 4L + 256j (fp32, j = 0..3) of the wave's 1024-element tile and reads the
// 8 or 4 codes of each slot directly (8 or 4 bytes, 512 or 256 bytes
// contiguous per load instruction; half that for 4-bit codes).
template <int B, typename Out, typename C = Int8Codes>
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
                float y[8];
                C::scaled8(codes, e, s, y);
                o.x = pack_bf16x2(y[0], y[1]);
                o.y = pack_bf16x2(y[2], y[3]);
                o.z = pack_bf16x2(y[4], y[5]);
                o.w = pack_bf16x2(y[6], y[7]);
            } else {
                float y[4];
                C::scaled4(codes, e, s, y);
                o.x = __builtin_bit_cast(uint32_t, y[0]);
                o.y = __builtin_bit_cast(uint32_t, y[1]);
                o.z = __builtin_bit_cast(uint32_t, y[2]);
                o.w = __builtin_bit_cast(uint32_t, y[3]);
            }
            store_b128(out + e, o);
        }
    }
}

// Row-bounded blocks with row_len % 16 == 0: each lane dequantizes the
// codes of one 16-byte output slot (8 bf16 or 4 fp32 elements), so that the
// lanes of a block store one contiguous range per instruction.  Against
// each lane storing its 16 elements directly (two or four 16-byte stores
// that each cover part of every line), on [8192, 2880], B = 256, µs: bf16
// 15.6 -> 14.2, fp32 81.0 -> 24.9 (B = 64, [8192, 2912], bf16: 16.5 ->
// 14.2), bit-identical.  Two slots per lane, 64 slots apart: bf16 15.5,
// fp32 26.0.
template <int B, int P>
struct RowSlots {
    size_t row_len, nblocks;
    uint32_t per_row;
    static constexpr int kLane = P;
    __device__ __forceinline__ LaneAt at(size_t g) const { return row_lane<B, P>(g, row_len, nblocks, per_row); }
};

template <int B, typename Out>
__global__ __launch_bounds__(kThreads) void k_dequantize_lanes(const int8_t* __restrict__ codes,
                                                               const float* __restrict__ scales,
                                                               RowSlots<B, 16 / sizeof(Out)> lanes,
                                                               Out* __restrict__ out, uint32_t ntiles) {
    constexpr int P = 16 / sizeof(Out);
    for (uint32_t tile = xcd_tile(blockIdx.x, gridDim.x); tile < ntiles; tile += gridDim.x) {
        const LaneAt a = lanes.at((size_t)tile * kThreads + threadIdx.x);
        if (!a.valid) continue;
        const float s = scales[a.blk];
        uint4 o;
        if constexpr (P == 8) {
            const uint2 w = load_b64(codes + a.e0);
            float y[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                y[k] = code_f32(w.x, k) * s;
                y[4 + k] = code_f32(w.y, k) * s;
            }
            o = make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                           pack_bf16x2(y[6], y[7]));
        } else {
            const uint32_t w = load_b32(codes + a.e0);
            o = make_uint4(__builtin_bit_cast(uint32_t, code_f32(w, 0) * s),
                           __builtin_bit_cast(uint32_t, code_f32(w, 1) * s),
                           __builtin_bit_cast(uint32_t, code_f32(w, 2) * s),
                           __builtin_bit_cast(uint32_t, code_f32(w, 3) * s));
        }
        store_b128(out + a.e0, o);
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
        for (int t = 0; t < kRowSlots; ++t) q[t] = (int8_t)(code_bits_of(fast_quotient(v[t], s, r)) & 0xFFu);
    } else if (s != 0.0f) {
#pragma unroll
        for (int t = 0; t < kRowSlots; ++t) q[t] = (int8_t)(clamped_code_bits_of(v[t] / s) & 0xFFu);
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

// Launches k<<<blocks, kThreads, 0, st>>>(a...) and returns that launch's
// own status.  hipLaunchKernel reports the launch it was asked for; reading
// hipGetLastError() after a triple-chevron launch would instead return any
// error an unrelated runtime call had left on the thread.
template <typename... P, typename... A>
hipError_t launch(void (*k)(P...), uint32_t blocks, hipStream_t st, A&&... a) {
    static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
    std::tuple<std::decay_t<P>...> vals(static_cast<std::decay_t<P>>(std::forward<A>(a))...);
    void* args[sizeof...(P)];
    std::apply([&](auto&... v) {
        size_t i = 0;
        ((args[i++] = static_cast<void*>(&v)), ...);
    }, vals);
    return hipLaunchKernel(reinterpret_cast<const void*>(k), dim3(blocks), dim3(kThreads), args, 0, st);
}

struct Grid {
    uint32_t ntiles, blocks;
};

// One workgroup per tile, at most `cap` workgroups (0: kMaxGrid); the
// kernels' grid-stride loops cover the rest.
Grid grid_for(size_t n, uint32_t cap = 0) {
    const size_t tiles = (n + kTileElems - 1) / kTileElems;
    const size_t limit = cap ? (cap < kMaxGrid ? cap : kMaxGrid) : kMaxGrid;
    Grid g;
    g.ntiles = (uint32_t)tiles;
    g.blocks = (uint32_t)(tiles < limit ? tiles : limit);
    return g;
}

Grid grid_lanes(size_t lanes) { return grid_for(lanes * kLaneElems); }

template <typename T>
struct TypeTag {
    using type = T;
};

// calls f(std::integral_constant<int, B>) for the supported block sizes
template <typename F>
hipError_t dispatch_block(int block, F&& f) {
    switch (block) {
    case 64: return f(std::integral_constant<int, 64>{});
    case 128: return f(std::integral_constant<int, 128>{});
    default: return f(std::integral_constant<int, 256>{});
    }
}

// calls f(std::integral_constant<int, OUT>) for an output kind
template <typename F>
hipError_t dispatch_out(int out_kind, F&& f) {
    if (out_kind == kOutBF16) return f(std::integral_constant<int, kOutBF16>{});
    if (out_kind == kOutF32) return f(std::integral_constant<int, kOutF32>{});
    return f(std::integral_constant<int, kOutNone>{});
}

// calls f(TypeTag<element type>) for an input kind
template <typename F>
hipError_t dispatch_in(int in_kind, F&& f) {
    if (in_kind == kInBF16) return f(TypeTag<uint16_t>{});
    return f(TypeTag<float>{});
}

// calls f(TypeTag<codes format>) for a code kind
template <typename F>
hipError_t dispatch_code(int code, F&& f) {
    if (code == kCodeE4M3) return f(TypeTag<E4M3Codes>{});
    if (code == kCodeInt4) return f(TypeTag<Int4Codes>{});
    return f(TypeTag<Int8Codes>{});
}

template <int B, typename Lanes, typename C = Int8Codes>
hipError_t quantize_b(const void* x, int in_kind, Lanes lanes, Grid g, int8_t* codes, float* scales,
                      hipStream_t st) {
    return dispatch_in(in_kind, [&](auto it) {
        using In = typename decltype(it)::type;
        return launch(k_quantize<B, In, Lanes, C>, g.blocks, st, static_cast<const In*>(x), lanes, codes, scales,
                      g.ntiles);
    });
}

// The reduce with 8 elements per lane (reduce_tiles8) for int8 and E4M3
// codes from 6 to 8 ranks, and from 4 with a fused output; 16 per lane for
// fewer ranks, for more, and for 4-bit codes.  Measured with B = 256, one
// launch per call, µs (16 -> 8 per lane), no output / bf16 output:
//   16.8M elements: N=1 9.7 -> 12.9 / 14.6 -> 17.3; N=3 14.0 -> 16.1 /
//     19.6 -> 19.8; N=4 16.1 -> 17.4 / 22.0 -> 21.6; N=6 21.3 -> 21.1 /
//     26.8 -> 26.1; N=8 26.7 -> 26.1 / 32.8 -> 31.6
//   8.4M: N=4 9.95 -> 10.54 / 13.47 -> 12.84; N=6 12.72 -> 12.46 / 15.75 ->
//     15.12; N=8 15.59 -> 15.12 / 18.33 -> 18.02
//   4.2M: N=6 8.12 -> 8.65 / 9.58 -> 9.97; N=8 9.96 -> 9.87 / 11.39 -> 11.43
//   2.1M: N=4 5.15 -> 4.83 / 5.24 -> 5.03; N=8 6.73 -> 6.08 / 6.90 -> 6.34
// Few ranks leave too little arithmetic per element to pay for the lane's
// fixed work twice as often.  With N = 16 (67M elements, B = 64) twice the
// load instructions per byte cost more than they give: 8 chunks over 4
// streams 202.9 -> 210.1.  4-bit codes (4 bytes per lane): 17.8 -> 21.0 at
// 16.8M elements.
constexpr int kMaxRanks8 = 8;

bool reduce_is_narrow(int code, int nranks, int out_kind) {
    return code != kCodeInt4 && nranks <= kMaxRanks8 && (nranks >= 6 || (out_kind != kOutNone && nranks >= 4));
}

template <int B, typename Lanes, typename C = Int8Codes>
hipError_t reduce_b(const RankPtrs& rp, int nranks, Lanes lanes, Grid g, int8_t* codes_out, float* scales_out,
                    void* out, int out_kind, hipStream_t st) {
    return dispatch_out(out_kind, [&](auto oc) {
        constexpr int OUT = decltype(oc)::value;
        return launch(k_reduce<B, OUT, Lanes, C>, g.blocks, st, rp, nranks, lanes, codes_out, scales_out, out,
                      g.ntiles, TileMap{0, 0, 1, 1});
    });
}

template <int B, typename Lanes, typename C = Int8Codes>
hipError_t ring_b(const int8_t* codes_in, const float* scales_in, const void* local, int in_kind, Lanes lanes,
                  Grid g, int8_t* codes_out, float* scales_out, hipStream_t st) {
    return dispatch_in(in_kind, [&](auto it) {
        using In = typename decltype(it)::type;
        return launch(k_ring_step<B, In, Lanes, C>, g.blocks, st, codes_in, scales_in, static_cast<const In*>(local),
                      lanes, codes_out, scales_out, g.ntiles);
    });
}

template <int B, typename C = Int8Codes>
hipError_t dequantize_b(const int8_t* codes, const float* scales, size_t n, void* out, int out_kind,
                        hipStream_t st) {
    const Grid g = grid_for(n);
    if (out_kind == kOutBF16)
        return launch(k_dequantize<B, uint16_t, C>, g.blocks, st, codes, scales, n, static_cast<uint16_t*>(out),
                      g.ntiles);
    return launch(k_dequantize<B, float, C>, g.blocks, st, codes, scales, n, static_cast<float*>(out), g.ntiles);
}

// RowLanes<B> or RowLanes8<B> of a row-bounded call, and its lane count
template <int B, typename RL>
RL row_lanes(const RowsCall& c, size_t& nlanes) {
    RL l;
    l.row_len = c.row_len;
    l.per_row = (uint32_t)((c.row_len + B - 1) / B);
    l.nblocks = c.rows * l.per_row;
    nlanes = l.nblocks * (B / RL::kLane);
    return l;
}

// row-bounded blocks, row_len % 16 == 0: the vector kernels on RowLanes.
// The reduce with a fused output takes 8 elements per lane (fp32 output: any
// rank count; bf16: from 3 ranks), where a lane's 8 results are one or two
// 16-byte stores that the wavefront's lanes write contiguously, instead of
// 16 per lane, whose two or four stores per lane each cover a part of every
// line.  Measured on [8192, 2880] bf16 data, B = 256 (the last block of a
// row 64 elements), µs, 16 -> 8 per lane, bit-identical:
//   fp32 out: N=1 83.7 -> 34.3; N=4 83.5 -> 44.5; N=8 91.0 -> 61.3;
//     N=16 128.2 -> 96.0
//   bf16 out: N=1 22.1 -> 25.4; N=2 25.7 -> 26.4; N=3 29.4 -> 28.5;
//     N=8 48.4 -> 47.0; N=16 84.4 -> 83.5 (B = 64, [8192, 2912], N=8:
//     49.8 -> 47.9)
//   no output: N=1 15.9 -> 20.7; N=8 38.9 -> 40.1; N=16 73.4 -> 77.2, so
//     it keeps 16 per lane.
bool rows_reduce_is_narrow(int nranks, int out_kind) {
    return out_kind == kOutF32 || (out_kind == kOutBF16 && nranks >= 3);
}

template <int B>
hipError_t rows_vector(const RowsCall& c, hipStream_t st) {
    size_t nlanes = 0;
    const RowLanes<B> l = row_lanes<B, RowLanes<B>>(c, nlanes);
    const Grid g = grid_lanes(nlanes);
    switch (c.op) {
    case kRowsQuantize:
        return quantize_b<B>(c.x, c.kind, l, g, c.codes_out, c.scales_out, st);
    case kRowsReduce: {
        const int out_kind = c.out ? (c.kind == kInBF16 ? kOutBF16 : kOutF32) : kOutNone;
        if (rows_reduce_is_narrow(c.nranks, out_kind)) {
            size_t nlanes8 = 0;
            const RowLanes8<B> l8 = row_lanes<B, RowLanes8<B>>(c, nlanes8);
            const Grid g8 = grid_lanes(nlanes8); // 256 lanes per tile at either width
            return dispatch_out(out_kind, [&](auto oc) {
                constexpr int OUT = decltype(oc)::value;
                return launch(k_reduce8_rows<B, OUT>, g8.blocks, st, c.rp, c.nranks, l8, c.codes_out, c.scales_out,
                              c.out, g8.ntiles);
            });
        }
        return reduce_b<B>(c.rp, c.nranks, l, g, c.codes_out, c.scales_out, c.out, out_kind, st);
    }
    case kRowsRingStep:
        return ring_b<B>(c.codes_in, c.scales_in, c.x, c.kind, l, g, c.codes_out, c.scales_out, st);
    default:
        return dispatch_in(c.kind, [&](auto ot) {
            using Out = typename decltype(ot)::type;
            using RS = RowSlots<B, 16 / sizeof(Out)>;
            size_t nslots = 0;
            const RS ls = row_lanes<B, RS>(c, nslots);
            const Grid gs = grid_lanes(nslots); // 256 lanes per tile
            return launch(k_dequantize_lanes<B, Out>, gs.blocks, st, c.codes_in, c.scales_in, ls,
                          static_cast<Out*>(c.out), gs.ntiles);
        });
    }
}

uint32_t row_grid(size_t nblocks) { return (uint32_t)((nblocks + kThreads / 64 - 1) / (kThreads / 64)); }

} // namespace

// ---------------------------------------------------------------------------
// static workspace of the no-allocation entry point
//
// One array per device, created when the code object is loaded there and
// kept until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address is looked up once per
// device (that device current) and only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[kStaticWorkspaceBytes];

namespace {
constexpr int kScratchDevices = 64;
std::once_flag g_scratch_once[kScratchDevices];
uint8_t* g_scratch_ptr[kScratchDevices];
hipError_t g_scratch_err[kScratchDevices];
} // namespace

hipError_t static_workspace(uint8_t** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? static_cast<uint8_t*>(p) : nullptr;
    });
    *ptr = g_scratch_ptr[dev];
    return g_scratch_err[dev];
}

hipError_t launch_rows(const RowsCall& c, hipStream_t st) {
    if (c.vector) {
        switch (c.block) {
        case 64: return rows_vector<64>(c, st);
        case 128: return rows_vector<128>(c, st);
        default: return rows_vector<256>(c, st);
        }
    }
    RowMap map;
    map.rows = c.rows;
    map.row_len = c.row_len;
    map.block = (uint32_t)c.block;
    map.per_row = (uint32_t)((c.row_len + c.block - 1) / c.block);
    const size_t nblocks = c.rows * map.per_row;
    const uint32_t grid = row_grid(nblocks);
    return dispatch_in(c.kind, [&](auto it) {
        using T = typename decltype(it)::type;
        switch (c.op) {
        case kRowsQuantize:
            return launch(k_quantize_rows<T>, grid, st, static_cast<const T*>(c.x), map, nblocks, c.codes_out,
                          c.scales_out);
        case kRowsDequantize:
            return launch(k_dequantize_rows<T>, grid, st, c.codes_in, c.scales_in, map, nblocks,
                          static_cast<T*>(c.out));
        case kRowsReduce:
            return launch(k_reduce_rows<T>, grid, st, c.rp, c.nranks, map, nblocks, c.codes_out, c.scales_out,
                          static_cast<T*>(c.out));
        default:
            return launch(k_ring_step_rows<T>, grid, st, c.codes_in, c.scales_in, static_cast<const T*>(c.x), map,
                          nblocks, c.codes_out, c.scales_out);
        }
    });
}

hipError_t launch_reduce_unquantized(const PlainPtrs& xp, int nranks, size_t n, int kind, void* out,
                                     hipStream_t st) {
    const Grid g = grid_for(n);
    return dispatch_in(kind, [&](auto it) {
        using T = typename decltype(it)::type;
        return launch(k_reduce_unquantized<T>, g.blocks, st, xp, nranks, n, static_cast<T*>(out), g.ntiles);
    });
}

hipError_t launch_quantize(const void* x, int in_kind, size_t n, int block, int8_t* codes, float* scales,
                           hipStream_t st, int code) {
    const Grid g = grid_for(n);
    return dispatch_code(code, [&](auto ct) {
        using C = typename decltype(ct)::type;
        return dispatch_block(block, [&](auto bc) {
            constexpr int B = decltype(bc)::value;
            // fp32 data in 16-byte slots; bf16 keeps 16 elements per lane
            // (its 32 bytes per lane measured faster than slots: 10.6
            // against 11.1 us for 16.8M elements)
            if (in_kind == kInF32)
                return launch(k_quantize_slots<B, float, C>, g.blocks, st, static_cast<const float*>(x), n, codes,
                              scales, g.ntiles);
            return quantize_b<B, FlatLanes<B>, C>(x, in_kind, FlatLanes<B>{n}, g, codes, scales, st);
        });
    });
}


// Super-tiles of 64 tiles dealt round-robin to the XCDs instead of one range
// per XCD, for reduces of at least 8 ranks over at least 2^25 elements.
// Probe, rank buffers in one allocation, µs (ranges -> super-tiles): N=8
// 44M 70.2 -> 64.2, 50M 74.8 -> 72.2; N=16 (B=256) 44M 132.0 -> 122.5;
// N=16 (B=64) 33.5M 99.6 -> 95.0, 67M 197.0 -> 189.3.  Smaller grids and
// fewer ranks do not gain: N=8 16.8M 26.0 -> 27.5, N=2 44M 25.5 -> 27.8,
// N=4 67M 57.0 -> 57.6, the 8.4M chunks of the small-block headline 199
// -> 205.  The chip's mapping of addresses to HBM channels is undocumented;
// this follows the measurements.
uint32_t reduce_super(int nranks, size_t n, uint32_t blocks) {
    constexpr uint32_t kSuper = 64;
    return nranks >= 8 && n >= ((size_t)1 << 25) && blocks % (8 * kSuper) == 0 ? kSuper : 0;
}

// The launch of a reduce over n elements in tiles of tile_elems: the whole
// of it, or one chunk of interleaved chunks (ChunkOf).  blocks == 0: this
// chunk has no runs.
struct ReduceGrid {
    uint32_t ntiles, blocks;
    TileMap map;
};

ReduceGrid reduce_grid(int nranks, size_t n, uint32_t tile_elems, ChunkOf chunk) {
    const size_t tiles = (n + tile_elems - 1) / tile_elems;
    ReduceGrid r;
    if (chunk.count > 1) {
        const uint32_t q = (uint32_t)(kChunkRunElems / tile_elems);
        const size_t runs = (tiles + q - 1) / q;
        const size_t mine = chunk.index < runs ? (runs - 1 - chunk.index) / chunk.count + 1 : 0;
        r.ntiles = (uint32_t)(mine * q);
        r.map = TileMap{0, chunk.index, chunk.count, q};
    } else {
        r.ntiles = (uint32_t)tiles;
        r.map = TileMap{0, 0, 1, 1};
    }
    r.blocks = r.ntiles < kMaxGrid ? r.ntiles : kMaxGrid;
    if (chunk.count <= 1) r.map.super = reduce_super(nranks, n, r.blocks);
    return r;
}

hipError_t launch_reduce(const RankPtrs& rp, int nranks, size_t n, int block, int8_t* codes_out,
                         float* scales_out, void* out, int out_kind, hipStream_t st, int code, ChunkOf chunk) {
    return dispatch_code(code, [&](auto ct) {
        using C = typename decltype(ct)::type;
        return dispatch_block(block, [&](auto bc) {
            constexpr int B = decltype(bc)::value;
            return dispatch_out(out_kind, [&](auto oc) {
                constexpr int OUT = decltype(oc)::value;
                if (reduce_is_narrow(code, nranks, OUT)) {
                    const ReduceGrid g = reduce_grid(nranks, n, kTileElems8, chunk);
                    if (g.blocks == 0) return hipSuccess;
                    return launch(k_reduce8<B, OUT, C>, g.blocks, st, rp, nranks, n, codes_out, scales_out, out,
                                  g.ntiles, g.map);
                }
                const ReduceGrid g = reduce_grid(nranks, n, kTileElems, chunk);
                if (g.blocks == 0) return hipSuccess;
                if (OUT == kOutNone && nranks > kMaxRanks8)
                    return launch(k_reduce<B, kOutNone, FlatLanes<B>, C, 16>, g.blocks, st, rp, nranks,
                                  FlatLanes<B>{n}, codes_out, scales_out, out, g.ntiles, g.map);
                return launch(k_reduce<B, OUT, FlatLanes<B>, C>, g.blocks, st, rp, nranks, FlatLanes<B>{n},
                              codes_out, scales_out, out, g.ntiles, g.map);
            });
        });
    });
}

// The one-kernel step with 8 elements per lane from 2^23 elements on, 16
// below, for int8 and E4M3 codes.  Measured with N = 8, B = 256, bf16 in and
// out (µs, 16 -> 8 per lane): 2M elements 6.94 -> 7.43; 4M 12.26 -> 12.47;
// 8M 21.0 -> 20.7; 16.8M 38.5 -> 37.4 (E4M3 39.7 -> 37.6).  The 4-bit step,
// bound by VALU issue, keeps 16 per lane: with 8 it issues 1.21 instead of
// 0.89 VALU instructions per element (SQ counters) for 28.7-30.0 against
// 29.1-29.2 µs.
constexpr size_t kStep8MinElems = (size_t)1 << 23;

hipError_t launch_quantize_reduce(const void* x_own, int in_kind, int own, const RankPtrs& rp, int nranks,
                                  size_t n, int block, int8_t* own_codes, float* own_scales, int8_t* codes_out,
                                  float* scales_out, void* out, int out_kind, hipStream_t st, int code) {
    const bool eight = n >= kStep8MinElems && code != kCodeInt4;
    const Grid g = grid_for(n);
    const uint32_t tiles8 = (uint32_t)((n + kTileElems8 - 1) / kTileElems8);
    const uint32_t blocks8 = tiles8 < kMaxGrid ? tiles8 : kMaxGrid;
    // super-tiles as for the plain reduce (reduce_super); measured on the
    // step, µs: N = 8 × 44M 98.0 -> 92.9, N = 16 × 44M 166.6 -> 149.5,
    // N = 8 × 67M 144.7 -> 138.5 (N = 8 × 16.8M, left in ranges: 37.8 -> 39.2)
    const uint32_t super = reduce_super(nranks, n, eight ? blocks8 : g.blocks);
    // dense loads unless the last group of 8 ranks has 1-4 of them
    const bool dense = nranks % 8 == 0 || nranks % 8 >= 5;
    return dispatch_code(code, [&](auto ct) {
        using C = typename decltype(ct)::type;
        return dispatch_block(block, [&](auto bc) {
            constexpr int B = decltype(bc)::value;
            const FlatLanes<B> lanes{n};
            return dispatch_out(out_kind, [&](auto oc) {
                constexpr int OUT = decltype(oc)::value;
                return dispatch_in(in_kind, [&](auto it) {
                    using In = typename decltype(it)::type;
                    const In* x = static_cast<const In*>(x_own);
                    if (eight) {
                        if (dense)
                            return launch(k_quantize_reduce8<B, OUT, In, C, true>, blocks8, st, x, own, own_codes,
                                          own_scales, rp, nranks, n, codes_out, scales_out, out, tiles8, super);
                        return launch(k_quantize_reduce8<B, OUT, In, C, false>, blocks8, st, x, own, own_codes,
                                      own_scales, rp, nranks, n, codes_out, scales_out, out, tiles8, super);
                    }
                    if (dense)
                        return launch(k_quantize_reduce<B, OUT, In, C, true>, g.blocks, st, x, own, own_codes,
                                      own_scales, rp, nranks, lanes, codes_out, scales_out, out, g.ntiles, super);
                    return launch(k_quantize_reduce<B, OUT, In, C, false>, g.blocks, st, x, own, own_codes,
                                  own_scales, rp, nranks, lanes, codes_out, scales_out, out, g.ntiles, super);
                });
            });
        });
    });
}

hipError_t launch_ring_step(const int8_t* codes_in, const float* scales_in, const void* local, int in_kind,
                            size_t n, int block, int8_t* codes_out, float* scales_out, hipStream_t st, int code) {
    const Grid g = grid_for(n);
    return dispatch_code(code, [&](auto ct) {
        using C = typename decltype(ct)::type;
        return dispatch_block(block, [&](auto bc) {
            constexpr int B = decltype(bc)::value;
            // as for the quantize: fp32 local data in slots, bf16 per lane
            // (the ring workload's step: 7.47 against 7.63 us in slots)
            if (in_kind == kInF32)
                return launch(k_ring_step_slots<B, float, C>, g.blocks, st, codes_in, scales_in,
                              static_cast<const float*>(local), n, codes_out, scales_out, g.ntiles);
            return ring_b<B, FlatLanes<B>, C>(codes_in, scales_in, local, in_kind, FlatLanes<B>{n}, g, codes_out,
                                              scales_out, st);
        });
    });
}

hipError_t launch_dequantize(const int8_t* codes, const float* scales, size_t n, int block, void* out,
                             int out_kind, hipStream_t st, int code) {
    return dispatch_code(code, [&](auto ct) {
        using C = typename decltype(ct)::type;
        return dispatch_block(block, [&](auto bc) {
            constexpr int B = decltype(bc)::value;
            return dequantize_b<B, C>(codes, scales, n, out, out_kind, st);
        });
    });
}

} // namespace qar
