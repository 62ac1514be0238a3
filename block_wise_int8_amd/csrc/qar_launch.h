// qar_launch.h -- internal interface between the C ABI (qar_api.cpp) and the
// kernel launchers (qar_kernels.hip).  Arguments reaching these functions
// have already been validated.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace qar {

constexpr int kMaxRanks = 32;

enum : int { kInBF16 = 0, kInF32 = 1 };
enum : int { kOutNone = -1, kOutBF16 = 0, kOutF32 = 1 };
// code format of the flat calls: int8 integers, FP8 E4M3 bytes, or 4-bit
// integers two per byte (the row-bounded path is int8 only)
enum : int { kCodeInt8 = 0, kCodeE4M3 = 1, kCodeInt4 = 2 };

// Rank pointers travel in the kernel's argument segment (512 bytes).
struct RankPtrs {
    const int8_t* codes[kMaxRanks];
    const float* scales[kMaxRanks];
};

struct PlainPtrs {
    const void* x[kMaxRanks];
};

// The row-bounded general path (one wavefront per block).
enum : int { kRowsQuantize = 0, kRowsDequantize = 1, kRowsReduce = 2, kRowsRingStep = 3 };
struct RowsCall {
    int op;
    bool vector;              // row_len % 16 == 0 and 16-byte aligned: the vector kernels
    int kind;                 // element type of x / out (kInBF16 or kInF32)
    size_t rows, row_len;
    int block;
    const void* x;            // quantize: input; ring step: local
    const int8_t* codes_in;   // dequantize, ring step
    const float* scales_in;
    RankPtrs rp;              // reduce
    int nranks;
    int8_t* codes_out;
    float* scales_out;
    void* out;                // dequantize; reduce (optional, may be null)
};
hipError_t launch_rows(const RowsCall& c, hipStream_t st);

hipError_t launch_reduce_unquantized(const PlainPtrs& xp, int nranks, size_t n, int kind, void* out,
                                     hipStream_t st);
hipError_t launch_quantize(const void* x, int in_kind, size_t n, int block, int8_t* codes, float* scales,
                           hipStream_t st, int code = kCodeInt8);
// A chunk of a reduce cut into `count` interleaved chunks: the element range
// is taken in runs of kChunkRunElems, and chunk `index` computes runs index,
// index + count, index + 2 count, ...  The pointers passed with it are those
// of the whole reduce, and n is the whole reduce's element count.
constexpr size_t kChunkRunElems = (size_t)1 << 18;
struct ChunkOf {
    uint32_t index, count;
};
// Number of runs of kChunkRunElems that n elements take (the most chunks a
// reduce of n elements can be cut into).
inline size_t chunk_runs(size_t n) { return (n + kChunkRunElems - 1) / kChunkRunElems; }

hipError_t launch_reduce(const RankPtrs& rp, int nranks, size_t n, int block, int8_t* codes_out,
                         float* scales_out, void* out, int out_kind, hipStream_t st, int code = kCodeInt8,
                         ChunkOf chunk = ChunkOf{0, 1});
hipError_t launch_quantize_reduce(const void* x_own, int in_kind, int own, const RankPtrs& rp, int nranks,
                                  size_t n, int block, int8_t* own_codes, float* own_scales, int8_t* codes_out,
                                  float* scales_out, void* out, int out_kind, hipStream_t st,
                                  int code = kCodeInt8);
hipError_t launch_ring_step(const int8_t* codes_in, const float* scales_in, const void* local, int in_kind,
                            size_t n, int block, int8_t* codes_out, float* scales_out, hipStream_t st,
                            int code = kCodeInt8);
// The static workspace (a device array of kStaticWorkspaceBytes per device,
// 256-byte aligned): its device address on the current device, looked up on
// the first call per device and cached.
constexpr size_t kStaticWorkspaceBytes = (size_t)64 << 20;
hipError_t static_workspace(uint8_t** ptr);

hipError_t launch_dequantize(const int8_t* codes, const float* scales, size_t n, int block, void* out,
                             int out_kind, hipStream_t st, int code = kCodeInt8);

} // namespace qar
