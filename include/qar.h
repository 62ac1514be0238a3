/*
 * qar.h -- C ABI of libqar: dynamic block-wise int8 quantization and
 * quantized reduction, one GPU's share of a quantized AllReduce, for AMD
 * Instinct MI355X (gfx950).
 *
 * The method is EQuARX ("EQuARX: Efficient Quantized AllReduce in XLA for
 * Distributed Machine Learning Acceleration"; page summary, section
 * "technical framework", steps 1-4; section "key design", item 1): the
 * tensor is cut into blocks, each block is quantized from BF16/FP32 to INT8
 * with a range found at run time, the AllReduce sums the quantized
 * contributions, and the result is dequantized back to the original type.
 * The pages leave the arithmetic open; libqar fixes it as follows, for every
 * call, bit for bit:
 *
 *   scale  s   = absmax / 127            one IEEE binary32 division
 *   code   q_i = 0 if s == 0, else clamp(rne(x_i / s), -127, 127)
 *                (x_i / s is the correctly rounded binary32 quotient; rne
 *                rounds to the nearest integer, ties to even; -128 is
 *                never produced)
 *   value  y_i = (float)q_i * s           one binary32 multiply
 *   bf16   round-to-nearest-even of the binary32 value
 *
 * All binary32 arithmetic rounds to nearest even with gradual underflow (no
 * flush to zero); multiplies and adds are never fused.
 *
 * Layout.  A buffer of n elements is nb = n / block consecutive blocks of
 * `block` elements (row-major flattening; for a [rows, hidden] tensor with
 * hidden % block == 0 the blocks run along the hidden dimension).  Codes are
 * int8[n] in element order; scales are a separate float[nb], one per block,
 * in block order.
 *
 * Conventions shared by every call:
 *   - Pointers are device pointers owned by the caller.  libqar never
 *     allocates, frees or synchronizes device memory at run time (its one
 *     static device array, the workspace of qar_allreduce_simulated_static,
 *     is part of the loaded code object).
 *   - Calls are asynchronous: work is enqueued on `stream` (a hipStream_t
 *     passed as void*; NULL is the default stream) and the call returns.
 *   - Arguments are checked before anything is enqueued.  A failed check
 *     returns a QAR_ERR_* status and enqueues nothing.  A failed launch
 *     returns QAR_ERR_HIP; qar_last_error() then names the HIP error.
 *   - n == 0 is a valid empty call: QAR_OK, nothing enqueued, no pointer is
 *     read.
 *   - Requirements (calls with a block argument): block is 64, 128 or 256;
 *     n % block == 0;
 *     n <= QAR_MAX_ELEMENTS; element and code pointers 16-byte aligned;
 *     scale pointers 4-byte aligned.
 *   - Inputs must be finite, and so must every binary32 sum a reduce or
 *     ring step forms (the sum of finite values can overflow).  Output for
 *     NaN or infinite input, or for an overflowed sum, is unspecified (it is
 *     not checked, for speed).
 *   - Output buffers must not overlap input buffers, except where a call
 *     says otherwise.  Partial overlap is rejected with QAR_ERR_INVALID_ARG.
 *   - Any block-aligned sub-range of a valid call (pointers advanced by
 *     k*block elements and k scales) is itself a valid call with the same
 *     results in that range.
 *   - Thread-safe.  Global state: the per-thread text behind
 *     qar_last_error(); a per-device pool of HIP events that the calls
 *     forking work onto side streams borrow while they enqueue (created on
 *     demand, one set per call in flight at once, never device memory); and
 *     the static workspace of qar_allreduce_simulated_static.
 */
#ifndef QAR_H
#define QAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums below are passed by value across the ABI.  A C caller may pass
 * any int in their place; compiled as C++ (the library itself) they take int
 * as their fixed underlying type, so every such value is a value of the type
 * and an unknown one reaches the argument checks (QAR_ERR_UNSUPPORTED or
 * QAR_ERR_INVALID_ARG) instead of being undefined before them.  In C an
 * enum is an int-sized integer type either way. */
#ifdef __cplusplus
#define QAR_ENUM_BASE : int
#else
#define QAR_ENUM_BASE
#endif

typedef enum qar_status QAR_ENUM_BASE {
    QAR_OK = 0,
    QAR_ERR_INVALID_ARG = 1, /* null pointer, n % block != 0, bad rank count, overlap */
    QAR_ERR_MISALIGNED = 2,  /* a pointer breaks the alignment rule above */
    QAR_ERR_UNSUPPORTED = 3, /* block size or dtype outside what is built */
    QAR_ERR_HIP = 4,         /* the HIP runtime refused a launch or call */
    QAR_ERR_CAPACITY = 5     /* the call needs more static workspace than QAR_STATIC_WORKSPACE_BYTES */
} qar_status;

typedef enum qar_dtype QAR_ENUM_BASE {
    QAR_BF16 = 0, /* bfloat16, stored as 16-bit patterns */
    QAR_F32 = 1   /* IEEE binary32 */
} qar_dtype;

#define QAR_MAX_RANKS 32
#define QAR_MAX_ELEMENTS ((size_t)1 << 40)
#define QAR_MAX_STREAMS 16

/*
 * Per-block dynamic quantization ("technical framework" steps 1-2; "key
 * design" item 1).
 *   x       [in]  n elements of `dtype`.
 *   codes   [out] int8[n].
 *   scales  [out] float[n / block].
 */
qar_status qar_quantize_blocks(const void* x, qar_dtype dtype, size_t n, uint32_t block,
                               int8_t* codes, float* scales, void* stream);

/*
 * One-shot N-way reduce of quantized contributions, then requantization of
 * the sum ("technical framework" step 3: the AllReduce works on the
 * quantized data; the error that summation builds up is the problem the
 * abstract and the "problem definition" section name).  For each element:
 *   acc = y_0;  acc = acc + y_r for r = 1 .. nranks-1  (binary32, rank order)
 * and the result is quantize(acc) per block.
 *   codes, scales  [in]  HOST arrays of nranks DEVICE pointers, rank order;
 *                        codes[r] is int8[n], scales[r] is float[n/block].
 *   nranks         1 .. QAR_MAX_RANKS.
 *   codes_out      [out] int8[n];  scales_out [out] float[n/block].  These
 *                  may be exactly the buffers of one input rank (in place).
 *   out            [out, optional] NULL, or n elements of out_dtype that
 *                  receive dequantize(codes_out, scales_out) -- step 4,
 *                  fused.  It is the requantized result, not the raw sum, so
 *                  that every rank of a real AllReduce dequantizes identical
 *                  bits.
 */
qar_status qar_reduce_quantized(const int8_t* const* codes, const float* const* scales,
                                uint32_t nranks, size_t n, uint32_t block,
                                int8_t* codes_out, float* scales_out,
                                void* out, qar_dtype out_dtype, void* stream);

/*
 * This rank's quantize fused into the reduce: the one-shot reduce in which
 * rank `own` contributes its unquantized buffer x_own.  x_own is quantized in
 * the same pass ("technical framework" step 2), its codes and scales are
 * written to codes[own] / scales[own] (what the peers receive), and those
 * same values enter the rank-order sum ("technical framework" step 3).
 * Results (codes[own], scales[own], codes_out, scales_out, out) are
 * bit-identical to qar_quantize_blocks(x_own -> codes[own], scales[own])
 * followed by qar_reduce_quantized; x_own is read once and codes[own] is
 * never read back.
 *   x_own        [in]  n elements of dtype (bf16 or fp32).
 *   own          0 .. nranks-1.
 *   codes, scales HOST arrays of nranks DEVICE pointers; entry own is an
 *                output, the others are inputs (as in qar_reduce_quantized).
 *   codes_out, scales_out, out, out_dtype  as in qar_reduce_quantized, but
 *                they may not be rank own's buffers.
 */
qar_status qar_quantize_reduce(const void* x_own, qar_dtype dtype, uint32_t own, int8_t* const* codes,
                               float* const* scales, uint32_t nranks, size_t n, uint32_t block,
                               int8_t* codes_out, float* scales_out, void* out, qar_dtype out_dtype,
                               void* stream);

/* Elements per run of the chunked calls' interleaved chunks. */
#define QAR_CHUNK_RUN_ELEMS (1u << 18)

/*
 * The same reduce as a pipeline of chunks over streams (the pages' deep
 * pipelining of communication and compute, "key innovations" item 2 and
 * "key design" item 3, taken on one GPU).  The elements are taken in runs
 * of QAR_CHUNK_RUN_ELEMS (the last run shorter; a run holds whole blocks)
 * and cut into `nchunks` interleaved chunks: chunk c computes runs c,
 * c + nchunks, c + 2 nchunks, ..., so the chunks that run at once read
 * neighbouring addresses.  Chunk c is enqueued on streams[c % nstreams]
 * behind whatever that stream already holds.  Nothing else is enqueued: no event, no wait.  The caller
 * orders the chunks after the producers of the inputs and before the
 * consumers of the outputs on every stream used (events, or by producing
 * and consuming on those streams).  Consecutive calls on the same streams
 * therefore overlap: a stream holds its chunk in flight and the next
 * call's behind it (double buffering), so one stream's kernel ramps up
 * while another's drains; two calls with the same n, nchunks and streams
 * give chunk c the same runs on the same stream.  Results are
 * bit-identical to qar_reduce_quantized for every nchunks and nstreams.
 *   nchunks   >= 1 (clipped to the number of runs).
 *   streams   HOST array of nstreams hipStream_t (as void*), 1 .. QAR_MAX_STREAMS;
 *             NULL (the default stream) is allowed; the first
 *             min(nchunks, nstreams) are used.
 */
qar_status qar_reduce_quantized_chunked(const int8_t* const* codes, const float* const* scales,
                                        uint32_t nranks, size_t n, uint32_t block,
                                        int8_t* codes_out, float* scales_out,
                                        void* out, qar_dtype out_dtype,
                                        uint32_t nchunks, void* const* streams, uint32_t nstreams);

/*
 * qar_reduce_quantized_chunked ordered as one operation on `stream`: the
 * chunks start after everything already enqueued on `stream`, and `stream`
 * waits for all of them.  A stream of `streams` that is `stream` itself
 * needs no event; every other one costs an event record and a wait at each
 * end of the call (on MI355X with ROCm 7 this fork and join cost tens of
 * microseconds per call, so a sequence of independent reduces is better
 * enqueued with qar_reduce_quantized_chunked between one fork and one
 * join).  The events come from a per-device pool (created on first use,
 * never device memory).  Results are bit-identical to qar_reduce_quantized.
 *   nchunks   >= 1 (clipped to the number of runs of QAR_CHUNK_RUN_ELEMS).
 *   streams   HOST array of nstreams hipStream_t (as void*),
 *             1 .. QAR_MAX_STREAMS; an entry may be NULL (the default
 *             stream) only when `stream` is NULL too, i.e. when it is the
 *             calling stream.
 */
qar_status qar_reduce_quantized_pipelined(const int8_t* const* codes, const float* const* scales,
                                          uint32_t nranks, size_t n, uint32_t block,
                                          int8_t* codes_out, float* scales_out,
                                          void* out, qar_dtype out_dtype,
                                          uint32_t nchunks, void* const* streams,
                                          uint32_t nstreams, void* stream);

/*
 * One ring step: dequantize the incoming quantized buffer, add this rank's
 * own unquantized values, requantize ("technical framework" step 3 taken as
 * a ring; the error accumulates over the N-1 steps):
 *   acc_i = y_in,i + x_local,i   (binary32), then quantize(acc) per block.
 *   codes_in, scales_in  [in]  int8[n], float[n/block].
 *   local                [in]  n elements of `dtype` (bf16 or fp32).
 *   codes_out, scales_out [out] int8[n], float[n/block]; may be exactly
 *                        codes_in / scales_in (in place).
 */
qar_status qar_ring_step(const int8_t* codes_in, const float* scales_in,
                         const void* local, qar_dtype dtype, size_t n, uint32_t block,
                         int8_t* codes_out, float* scales_out, void* stream);

/*
 * Dequantize back to the original type ("technical framework" step 4):
 *   out_i = (float)q_i * s_b, stored as binary32 or rounded to bf16.
 *   codes, scales  [in]  int8[n], float[n/block].
 *   out            [out] n elements of out_dtype.
 */
qar_status qar_dequantize(const int8_t* codes, const float* scales, size_t n, uint32_t block,
                          void* out, qar_dtype out_dtype, void* stream);

/*
 * The comparator the pages measure against: the same N-way reduction on the
 * unquantized data (EQuARX abstract: the 1.8x is over a BF16 AllReduce).
 * For each element the binary32 sum of the ranks' values in rank order,
 * stored in the input type (bf16: rounded to nearest even).
 *   x       [in]  HOST array of nranks DEVICE pointers, each n elements of
 *                 dtype, rank order.
 *   nranks  1 .. QAR_MAX_RANKS.
 *   n       any multiple of 16 (no block structure).
 *   out     [out] n elements of dtype; may be exactly one input buffer.
 */
qar_status qar_reduce_unquantized(const void* const* x, uint32_t nranks, size_t n, qar_dtype dtype,
                                  void* out, void* stream);

/*
 * The whole quantized AllReduce of N rank buffers, simulated on one GPU:
 * the result every rank of a real AllReduce would hold, computed with the
 * calls above ("technical framework" steps 1-4, pipelined over chunks as in
 * "key innovations" item 2).  The buffer is cut into `nchunks` block-aligned
 * chunks; chunk c runs on streams[c % nstreams]:
 *   QAR_SCHEDULE_ONE_SHOT: every rank's chunk is quantized
 *     (codes_work[r], scales_work[r]), then one fused reduce in rank order
 *     0..N-1 requantizes the sum in place into codes_work[0]/scales_work[0]
 *     and writes its dequantized value to out.  The last rank's quantize
 *     runs inside that reduce (qar_quantize_reduce) when N > 1; the results
 *     are the same bits.  With nchunks = N the chunks are the N slices of a
 *     two-shot AllReduce's reduce-scatter (the TACO page, section 2.B
 *     item 3, kernel fusion and overlap: reduce-scatter, then all-gather); its
 *     all-gather forwards the requantized codes unchanged.
 *   QAR_SCHEDULE_RING: chunk c starts at rank s = c mod N, as the chunk
 *     rank s injects first in a ring: quantize(x_s), then ring steps adding
 *     x_{s+1}, ..., x_{s+N-1} (ranks mod N) in place in codes_work[0] /
 *     scales_work[0], then dequantize to out.  With nchunks = N this is the
 *     classic ring's reduce-scatter order; the all-gather forwards codes
 *     unchanged, so it adds no error and is not simulated.
 *   x            [in]  HOST array of nranks DEVICE pointers, n elements of dtype.
 *   codes_work, scales_work  HOST arrays of DEVICE pointers: int8[n] and
 *                float[n/block] workspaces; nranks of each for ONE_SHOT, only
 *                [0] is used for RING (the rest may be NULL).
 *   out          [out] n elements of dtype.
 *   nchunks      >= 1 (clipped to the number of blocks); streams: HOST array
 *                of 1..QAR_MAX_STREAMS handles (NULL only when `stream` is
 *                NULL); `stream` orders the whole call as in
 *                qar_reduce_quantized_pipelined.
 * Results are bit-identical for every nchunks and nstreams under ONE_SHOT;
 * under RING they depend on nchunks through each chunk's starting rank.
 */
typedef enum qar_schedule QAR_ENUM_BASE { QAR_SCHEDULE_ONE_SHOT = 0, QAR_SCHEDULE_RING = 1 } qar_schedule;

qar_status qar_allreduce_simulated(const void* const* x, qar_dtype dtype, uint32_t nranks, size_t n,
                                   uint32_t block, qar_schedule schedule, int8_t* const* codes_work,
                                   float* const* scales_work, void* out, uint32_t nchunks,
                                   void* const* streams, uint32_t nstreams, void* stream);

/*
 * For callers that cannot allocate: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  qar_allreduce_simulated
 * with the same arguments minus the workspaces and the side streams: every
 * chunk runs on `stream` in chunk order, and the per-rank code and scale
 * staging lives in a static device array inside libqar,
 * QAR_STATIC_WORKSPACE_BYTES per device, held by every device the library
 * runs on until the process ends.  The call allocates nothing, records no
 * event and synchronizes nothing; results are bit-identical to
 * qar_allreduce_simulated with the same schedule and nchunks.
 *   Capacity: one-shot stages nranks * (n + 4 n/block) bytes, the ring
 *   n + 4 n/block (each rounded up to 256 bytes per rank and array); a
 *   call that needs more returns QAR_ERR_CAPACITY and enqueues nothing
 *   (qar_last_error() gives the sizes).
 *   Sharing: all calls on one device use the same array.  Calls whose work
 *   overlaps in time on one device (on different streams, or from several
 *   threads without ordering between their streams) race on it; order them
 *   on one stream or with events.  Nothing in the array needs to start at
 *   zero: every byte a call reads there was written earlier by that call.
 *   The device address of the array is looked up on the first call per
 *   device (hipGetSymbolAddress) and cached.
 */
#define QAR_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)

qar_status qar_allreduce_simulated_static(const void* const* x, qar_dtype dtype, uint32_t nranks, size_t n,
                                          uint32_t block, qar_schedule schedule, void* out, uint32_t nchunks,
                                          void* stream);

/*
 * Row-bounded blocks: the same four operations on a [rows, row_len] tensor
 * whose block grid restarts at every row, so the last block of a row holds
 * row_len % block elements when row_len is not a multiple of block (a block
 * never spans two rows).  Each row has per_row = ceil(row_len / block)
 * blocks; scales hold rows * per_row values, row-major; codes and data hold
 * rows * row_len elements, row-major.  The arithmetic of every block is that
 * of the calls above, a partial block taking its absmax over its own
 * elements.  When row_len % block == 0 the block grids coincide and the call
 * is exactly the flat call with n = rows * row_len.
 * Requirements: block 64, 128 or 256; rows * row_len <= QAR_MAX_ELEMENTS;
 * rows * per_row <= QAR_MAX_ROW_BLOCKS; data pointers aligned to their
 * element size, scales to 4 bytes, codes unconstrained (the flat fast path
 * is taken when the flat call's 16-byte alignment also holds).
 */
#define QAR_MAX_ROW_BLOCKS ((size_t)1 << 26)

qar_status qar_quantize_rows(const void* x, qar_dtype dtype, size_t rows, size_t row_len, uint32_t block,
                             int8_t* codes, float* scales, void* stream);
qar_status qar_reduce_quantized_rows(const int8_t* const* codes, const float* const* scales, uint32_t nranks,
                                     size_t rows, size_t row_len, uint32_t block, int8_t* codes_out,
                                     float* scales_out, void* out, qar_dtype out_dtype, void* stream);
qar_status qar_ring_step_rows(const int8_t* codes_in, const float* scales_in, const void* local, qar_dtype dtype,
                              size_t rows, size_t row_len, uint32_t block, int8_t* codes_out, float* scales_out,
                              void* stream);
qar_status qar_dequantize_rows(const int8_t* codes, const float* scales, size_t rows, size_t row_len,
                               uint32_t block, void* out, qar_dtype out_dtype, void* stream);

/*
 * FP8 E4M3 codes.  The same calls with 8-bit floating-point codes in place
 * of int8 integers: the format the TACO page argues for ("TACO: Efficient
 * Communication Compression of Intermediate Tensors for Scalable
 * Tensor-Parallel LLM Training", page summary in Dutch, section 2.A "Waarom
 * FP8?", why FP8), with the per-block scale of its section 2.B item 2
 * "Dual-Scale (DS) Quantization" that brings the block into FP8's range Q_max (only
 * that scale; no rotation).  E4M3 is the OCP format: sign, 4 exponent bits
 * with bias 7, 3 mantissa bits, subnormals (m/8) * 2^-6, no infinity, codes
 * 0x7F and 0xFF NaN (never produced), largest finite value 448.
 *
 *   scale  s   = absmax / 448            one IEEE binary32 division
 *   code   c_i = 0x00 if s == 0; else the E4M3 value nearest to
 *                clamp(x_i / s, -448, 448) (the correctly rounded binary32
 *                quotient), ties to the even mantissa; the sign is kept, so
 *                a negative quotient that rounds to zero gives 0x80 (-0)
 *   value  y_i = e4m3(c_i) * s           one binary32 multiply
 *
 * Codes are uint8_t[n], one byte per element, in the same layout as the int8
 * codes; scales, alignment, aliasing, streams and errors are exactly those of
 * the int8 call of the same name.  The reduce, the one-kernel step and the
 * ring step sum in binary32 in rank order and requantize with this
 * quantizer; a sum is -0 only when every term is.
 */
qar_status qar_quantize_blocks_e4m3(const void* x, qar_dtype dtype, size_t n, uint32_t block, uint8_t* codes,
                                    float* scales, void* stream);
qar_status qar_reduce_quantized_e4m3(const uint8_t* const* codes, const float* const* scales, uint32_t nranks,
                                     size_t n, uint32_t block, uint8_t* codes_out, float* scales_out, void* out,
                                     qar_dtype out_dtype, void* stream);
qar_status qar_quantize_reduce_e4m3(const void* x_own, qar_dtype dtype, uint32_t own, uint8_t* const* codes,
                                    float* const* scales, uint32_t nranks, size_t n, uint32_t block,
                                    uint8_t* codes_out, float* scales_out, void* out, qar_dtype out_dtype,
                                    void* stream);
qar_status qar_ring_step_e4m3(const uint8_t* codes_in, const float* scales_in, const void* local,
                              qar_dtype dtype, size_t n, uint32_t block, uint8_t* codes_out, float* scales_out,
                              void* stream);
qar_status qar_dequantize_e4m3(const uint8_t* codes, const float* scales, size_t n, uint32_t block, void* out,
                               qar_dtype out_dtype, void* stream);

/*
 * 4-bit integer codes.  The same calls with 4-bit codes, two per byte.  The
 * pages name 4-bit communication quantization only through titles in their
 * reference lists (SDP4Bit; Echo, error-compensated 4-bit tensor-parallel
 * communication); libqar takes the int8 method at 4 bits:
 *
 *   scale  s   = absmax / 7              one IEEE binary32 division
 *   code   q_i = 0 if s == 0, else clamp(rne(x_i / s), -7, 7)
 *   value  y_i = (float)q_i * s
 *
 * Codes are packed: element 2k in the low nibble of byte k, element 2k+1 in
 * the high nibble, two's complement (-8 is never produced); a buffer of n
 * elements takes n/2 bytes.  A block-aligned sub-range starts block/2 bytes
 * per block into the codes.  Alignment, aliasing (in place: the whole packed
 * buffer and the scales), streams and errors are those of the int8 call of
 * the same name; sizes of code buffers are n/2 bytes instead of n.
 */
qar_status qar_quantize_blocks_int4(const void* x, qar_dtype dtype, size_t n, uint32_t block, uint8_t* codes,
                                    float* scales, void* stream);
qar_status qar_reduce_quantized_int4(const uint8_t* const* codes, const float* const* scales, uint32_t nranks,
                                     size_t n, uint32_t block, uint8_t* codes_out, float* scales_out, void* out,
                                     qar_dtype out_dtype, void* stream);
qar_status qar_quantize_reduce_int4(const void* x_own, qar_dtype dtype, uint32_t own, uint8_t* const* codes,
                                    float* const* scales, uint32_t nranks, size_t n, uint32_t block,
                                    uint8_t* codes_out, float* scales_out, void* out, qar_dtype out_dtype,
                                    void* stream);
qar_status qar_ring_step_int4(const uint8_t* codes_in, const float* scales_in, const void* local,
                              qar_dtype dtype, size_t n, uint32_t block, uint8_t* codes_out, float* scales_out,
                              void* stream);
qar_status qar_dequantize_int4(const uint8_t* codes, const float* scales, size_t n, uint32_t block, void* out,
                               qar_dtype out_dtype, void* stream);

/* Static text for a status code. */
const char* qar_status_string(qar_status status);

/* Text of the last QAR_ERR_HIP raised on the calling thread ("" if none). */
const char* qar_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QAR_H */
