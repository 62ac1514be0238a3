/*
 * qar_oracle.c -- plain, slow CPU oracle for dynamic block-wise int8
 * quantization and quantized reduction.
 *
 * TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
 * CPU-baseline leg load this file's shared object; the library under
 * block_wise_int8_amd/ never does, and this file shares no code, header or
 * constant with it.
 *
 * What it follows.  "EQuARX: Efficient Quantized AllReduce in XLA for
 * Distributed Machine Learning Acceleration" (page summary on shd-paper.top):
 *   - section "technical framework", step 1: the input is cut into blocks;
 *   - step 2: each block is quantized dynamically from BF16 or FP32 to INT8;
 *   - step 3: the AllReduce runs on the quantized data (the summation is
 *     where error builds up: same page, "problem definition", and the
 *     abstract);
 *   - step 4: the result is dequantized back to the original type;
 *   - section "key design", item 1: each block's range is found at run time.
 * The pages leave the arithmetic open.  The readings taken here:
 *   scale  s   = fl32(absmax / 127)            one IEEE fp32 division
 *   code   q_i = 0                              if s == 0
 *              = clamp(rne(fl32(x_i / s)), -127, 127)   otherwise
 *   value  y_i = fl32((float)q_i * s)           dequantize
 *   reduce acc = y_0, then acc = fl32(acc + y_r) for r = 1..N-1 (rank
 *          order, separate multiply and add), then quantize(acc)
 *   ring   quantize(fl32(y_in + x_local))
 *   bf16   round-to-nearest-even of the fp32 value to 8 significant bits.
 * Inputs must be finite; the oracle refuses NaN and infinity, and refuses a
 * reduce or ring step whose binary32 sum overflows to infinity.
 *
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -fPIC -shared.
 * x86-64 SSE arithmetic (FLT_EVAL_METHOD == 0): every float operation below
 * rounds once to binary32, round-to-nearest-even, with gradual underflow.
 *
 * Every function works on host memory, any block length >= 1, and a
 * partial last block (its absmax covers only its own elements).
 */
#include <float.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if FLT_EVAL_METHOD != 0
#error "the oracle needs binary32 evaluation of float expressions"
#endif

enum { ORACLE_BF16 = 0, ORACLE_F32 = 1 };
enum { ORACLE_OK = 0, ORACLE_BAD_ARG = -1, ORACLE_NONFINITE = -2 };

/* bf16 is the top half of a binary32 word, so widening is exact. */
static float bf16_bits_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a finite binary32 value to the nearest bfloat16, ties to the even
 * neighbour.  The magnitude bits are rounded; the sign bit rides along. */
static uint16_t float_to_bf16_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t upper = u >> 16;        /* truncated bf16 pattern          */
    uint32_t rest = u & 0xFFFFu;     /* dropped low half of the pattern */
    if (rest > 0x8000u || (rest == 0x8000u && (upper & 1u)))
        upper += 1u;                 /* carries into the exponent as IEEE does */
    return (uint16_t)upper;
}

static float load_element(const void* x, int dtype, size_t i)
{
    if (dtype == ORACLE_BF16)
        return bf16_bits_to_float(((const uint16_t*)x)[i]);
    return ((const float*)x)[i];
}

/* Quantize one block of `len` fp32 values: writes len codes and one scale. */
static void quantize_one_block(const float* v, size_t len, int8_t* q, float* scale)
{
    float absmax = 0.0f;
    for (size_t i = 0; i < len; i++) {
        float m = fabsf(v[i]);
        if (m > absmax)
            absmax = m;
    }
    float s = absmax / 127.0f;
    *scale = s;
    for (size_t i = 0; i < len; i++) {
        if (s == 0.0f) {
            q[i] = 0;
            continue;
        }
        float t = v[i] / s;
        float r = nearbyintf(t); /* default rounding mode: to nearest, ties even */
        if (r > 127.0f)
            r = 127.0f;
        if (r < -127.0f)
            r = -127.0f;
        q[i] = (int8_t)r;
    }
}

/* A sum of finite values can still overflow binary32; such a block has no
 * finite absmax and the method is undefined there, so the oracle refuses it
 * as it refuses non-finite input. */
static int all_finite(const float* v, size_t len)
{
    for (size_t i = 0; i < len; i++)
        if (!isfinite(v[i]))
            return 0;
    return 1;
}

static size_t block_count(size_t n, size_t block) { return (n + block - 1) / block; }

static float dequant_value(int8_t q, float s) { return (float)q * s; }

/* x: n elements of dtype (bf16 as raw uint16 patterns, or fp32).
 * codes: int8[n]; scales: fp32[ceil(n / block)]. */
int oracle_quantize(const void* x, int dtype, size_t n, size_t block,
                    int8_t* codes, float* scales)
{
    if (block == 0 || (dtype != ORACLE_BF16 && dtype != ORACLE_F32))
        return ORACLE_BAD_ARG;
    if (n == 0)
        return ORACLE_OK;
    if (!x || !codes || !scales)
        return ORACLE_BAD_ARG;
    for (size_t i = 0; i < n; i++)
        if (!isfinite(load_element(x, dtype, i)))
            return ORACLE_NONFINITE;
    float* v = malloc(block * sizeof *v);
    if (!v)
        return ORACLE_BAD_ARG;
    size_t nb = block_count(n, block);
    for (size_t b = 0; b < nb; b++) {
        size_t start = b * block;
        size_t len = (n - start < block) ? n - start : block;
        for (size_t i = 0; i < len; i++)
            v[i] = load_element(x, dtype, start + i);
        quantize_one_block(v, len, codes + start, scales + b);
    }
    free(v);
    return ORACLE_OK;
}

/* out: fp32[n] = (float)code * scale of its block. */
int oracle_dequantize_f32(const int8_t* codes, const float* scales, size_t n,
                          size_t block, float* out)
{
    if (block == 0)
        return ORACLE_BAD_ARG;
    for (size_t i = 0; i < n; i++)
        out[i] = dequant_value(codes[i], scales[i / block]);
    return ORACLE_OK;
}

/* out: bf16[n] patterns, the fp32 dequantized value rounded to bf16. */
int oracle_dequantize_bf16(const int8_t* codes, const float* scales, size_t n,
                           size_t block, uint16_t* out)
{
    if (block == 0)
        return ORACLE_BAD_ARG;
    for (size_t i = 0; i < n; i++)
        out[i] = float_to_bf16_bits(dequant_value(codes[i], scales[i / block]));
    return ORACLE_OK;
}

/* One-shot N-way reduce.  codes[r] / scales[r] hold rank r's quantized
 * buffer (n codes, ceil(n/block) scales).  Each element is the fp32 sum of
 * the dequantized contributions taken in rank order 0, 1, ..., N-1; the sum
 * is then quantized again per block. */
int oracle_reduce(const int8_t* const* codes, const float* const* scales,
                  size_t nranks, size_t n, size_t block,
                  int8_t* codes_out, float* scales_out)
{
    if (block == 0 || nranks == 0)
        return ORACLE_BAD_ARG;
    if (n == 0)
        return ORACLE_OK;
    float* acc = malloc(block * sizeof *acc);
    if (!acc)
        return ORACLE_BAD_ARG;
    size_t nb = block_count(n, block);
    for (size_t b = 0; b < nb; b++) {
        size_t start = b * block;
        size_t len = (n - start < block) ? n - start : block;
        for (size_t i = 0; i < len; i++)
            acc[i] = dequant_value(codes[0][start + i], scales[0][b]);
        for (size_t r = 1; r < nranks; r++)
            for (size_t i = 0; i < len; i++)
                acc[i] = acc[i] + dequant_value(codes[r][start + i], scales[r][b]);
        if (!all_finite(acc, len)) {
            free(acc);
            return ORACLE_NONFINITE;
        }
        quantize_one_block(acc, len, codes_out + start, scales_out + b);
    }
    free(acc);
    return ORACLE_OK;
}

/* One ring step: dequantize the incoming buffer, add this rank's own
 * unquantized values (bf16 or fp32), quantize the sum per block. */
int oracle_ring_step(const int8_t* codes_in, const float* scales_in,
                     const void* local, int dtype, size_t n, size_t block,
                     int8_t* codes_out, float* scales_out)
{
    if (block == 0 || (dtype != ORACLE_BF16 && dtype != ORACLE_F32))
        return ORACLE_BAD_ARG;
    if (n == 0)
        return ORACLE_OK;
    for (size_t i = 0; i < n; i++)
        if (!isfinite(load_element(local, dtype, i)))
            return ORACLE_NONFINITE;
    float* acc = malloc(block * sizeof *acc);
    if (!acc)
        return ORACLE_BAD_ARG;
    size_t nb = block_count(n, block);
    for (size_t b = 0; b < nb; b++) {
        size_t start = b * block;
        size_t len = (n - start < block) ? n - start : block;
        for (size_t i = 0; i < len; i++)
            acc[i] = dequant_value(codes_in[start + i], scales_in[b]) +
                     load_element(local, dtype, start + i);
        if (!all_finite(acc, len)) {
            free(acc);
            return ORACLE_NONFINITE;
        }
        quantize_one_block(acc, len, codes_out + start, scales_out + b);
    }
    free(acc);
    return ORACLE_OK;
}

/* The comparator of the method: the same N-way reduction on the
 * unquantized data (EQuARX abstract: the speed-up is measured against a
 * BF16 AllReduce).  Each element is the binary32 sum of the N ranks' values
 * in rank order, stored in the input type (bf16: rounded to nearest even).
 * x[r]: rank r's n elements of dtype; out: n elements of dtype. */
int oracle_reduce_unquantized(const void* const* x, int dtype, size_t nranks, size_t n, void* out)
{
    if (nranks == 0 || (dtype != ORACLE_BF16 && dtype != ORACLE_F32))
        return ORACLE_BAD_ARG;
    for (size_t r = 0; r < nranks; r++)
        for (size_t i = 0; i < n; i++)
            if (!isfinite(load_element(x[r], dtype, i)))
                return ORACLE_NONFINITE;
    for (size_t i = 0; i < n; i++) {
        float acc = load_element(x[0], dtype, i);
        for (size_t r = 1; r < nranks; r++)
            acc = acc + load_element(x[r], dtype, i);
        if (!isfinite(acc))
            return ORACLE_NONFINITE;
        if (dtype == ORACLE_BF16)
            ((uint16_t*)out)[i] = float_to_bf16_bits(acc);
        else
            ((float*)out)[i] = acc;
    }
    return ORACLE_OK;
}

/* The bf16 rounding on its own, so that tests can pin it to a library
 * conversion. */
void oracle_f32_to_bf16(const float* in, size_t n, uint16_t* out)
{
    for (size_t i = 0; i < n; i++)
        out[i] = float_to_bf16_bits(in[i]);
}

/* ------------------------------------------------------------------------
 * FP8 E4M3 codes: the same block-wise method with 8-bit floating-point codes
 * instead of integers.  "TACO: Efficient Communication Compression of
 * Intermediate Tensors for Scalable Tensor-Parallel LLM Training" (page
 * summary, in Dutch), section 2.A "Waarom FP8?" (why FP8): the E4M3 format's
 * exponential spacing keeps precision for the many small values and range
 * for the outliers; section 2.B item 2, "Dual-Scale (DS) Quantization": a per-block scale
 * brings the block into FP8's dynamic range, Q_max.  Only that single
 * post-scale is taken here (no rotation, no pre-scale).
 *
 * E4M3 as defined by the OCP 8-bit floating point specification: sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
 * subnormals m/8 * 2^-6; exponent field 15 with mantissa 7 is NaN and there
 * is no infinity, so the largest finite value is 1.75 * 2^8 = 448 (Q_max).
 *
 * Readings:
 *   scale  s   = fl32(absmax / 448)
 *   code   c_i = 0x00                                        if s == 0
 *              = E4M3 nearest to clamp(fl32(x_i / s), -448, 448), ties to
 *                the even code; the sign is kept, so a negative quotient
 *                that rounds to zero gives 0x80 (-0)
 *   value  y_i = fl32(e4m3(c_i) * s)
 *   reduce and ring: as for int8 codes, with this quantizer and value.
 * ------------------------------------------------------------------------ */

#define E4M3_MAX 448.0f

/* The value of an E4M3 code, from the format's definition (NaN codes give
 * NaN). */
static float e4m3_value(uint8_t c)
{
    int e = (c >> 3) & 15;
    int m = c & 7;
    float mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexpf((float)m, -9);                 /* (m/8) * 2^-6 */
    else
        mag = ldexpf((float)(8 + m), e - 10);       /* (1 + m/8) * 2^(e-7) */
    return (c & 0x80) ? -mag : mag;
}

/* The non-negative finite E4M3 values in code order 0..126, which is
 * increasing order; filled from e4m3_value() when the library is loaded. */
static float e4m3_table[127];

__attribute__((constructor)) static void e4m3_fill_table(void)
{
    for (unsigned c = 0; c < 127; c++)
        e4m3_table[c] = e4m3_value((uint8_t)c);
}

/* The E4M3 code nearest to t, |t| <= 448, ties to the code whose mantissa
 * (lowest bit) is even.  Binary search in the ordered table for the largest
 * value <= |t|, then the nearer of it and the next one; both distances are
 * exact in binary64. */
static uint8_t e4m3_nearest(float t)
{
    uint8_t sign = signbit(t) ? 0x80 : 0x00;
    float a = fabsf(t);
    unsigned lo = 0, hi = 126;           /* invariant: table[lo] <= a */
    while (lo < hi) {
        unsigned mid = (lo + hi + 1) / 2;
        if (e4m3_table[mid] <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    unsigned c = lo;
    if (c < 126) {
        double below = (double)a - (double)e4m3_table[c];
        double above = (double)e4m3_table[c + 1] - (double)a;
        if (above < below || (above == below && (c & 1u)))
            c++;
    }
    return (uint8_t)(sign | c);
}

static void quantize_one_block_e4m3(const float* v, size_t len, uint8_t* q, float* scale)
{
    float absmax = 0.0f;
    for (size_t i = 0; i < len; i++) {
        float m = fabsf(v[i]);
        if (m > absmax)
            absmax = m;
    }
    float s = absmax / E4M3_MAX;
    *scale = s;
    for (size_t i = 0; i < len; i++) {
        if (s == 0.0f) {
            q[i] = 0x00;
            continue;
        }
        float t = v[i] / s;
        if (t > E4M3_MAX)
            t = E4M3_MAX;
        if (t < -E4M3_MAX)
            t = -E4M3_MAX;
        q[i] = e4m3_nearest(t);
    }
}

static float dequant_value_e4m3(uint8_t c, float s) { return e4m3_value(c) * s; }

/* x: n elements of dtype; codes: E4M3 bytes[n]; scales: fp32[ceil(n/block)]. */
int oracle_quantize_e4m3(const void* x, int dtype, size_t n, size_t block,
                         uint8_t* codes, float* scales)
{
    if (block == 0 || (dtype != ORACLE_BF16 && dtype != ORACLE_F32))
        return ORACLE_BAD_ARG;
    if (n == 0)
        return ORACLE_OK;
    if (!x || !codes || !scales)
        return ORACLE_BAD_ARG;
    for (size_t i = 0; i < n; i++)
        if (!isfinite(load_element(x, dtype, i)))
            return ORACLE_NONFINITE;
    float* v = malloc(block * sizeof *v);
    if (!v)
        return ORACLE_BAD_ARG;
    size_t nb = block_count(n, block);
    for (size_t b = 0; b < nb; b++) {
        size_t start = b * block;
        size_t len = (n - start < block) ? n - start : block;
        for (size_t i = 0; i < len; i++)
            v[i] = load_element(x, dtype, start + i);
        quantize_one_block_e4m3(v, len, codes + start, scales + b);
    }
    free(v);
    return ORACLE_OK;
}

/* out: fp32[n] (out_dtype ORACLE_F32) or bf16 patterns (ORACLE_BF16). */
int oracle_dequantize_e4m3(const uint8_t* codes, const float* scales, size_t n,
                           size_t block, int out_dtype, void* out)
{
    if (block == 0 || (out_dtype != ORACLE_BF16 && out_dtype != ORACLE_F32))
        return ORACLE_BAD_ARG;
    for (size_t i = 0; i < n; i++) {
        float y = dequant_value_e4m3(codes[i], scales[i / block]);
        if (out_dtype == ORACLE_BF16)
            ((uint16_t*)out)[i] = float_to_bf16_bits(y);
        else
            ((float*)out)[i] = y;
    }
    return ORACLE_OK;
}

/* One-shot N-way reduce of E4M3-coded ranks, rank order 0..N-1. */
int oracle_reduce_e4m3(const uint8_t* const* codes, const float* const* scales,
                       size_t nranks, size_t n, size_t block,
                       uint8_t* codes_out, float* scales_out)
{
    if (block == 0 || nranks == 0)
        return ORACLE_BAD_ARG;
    if (n == 0)
        return ORACLE_OK;
    float* acc = malloc(block * sizeof *acc);
    if (!acc)
        return ORACLE_BAD_ARG;
    size_t nb = block_count(n, block);
    for (size_t b = 0; b < nb; b++) {
        size_t start = b * block;
        size_t len = (n - start < block) ? n - start : block;
        for (size_t i = 0; i < len; i++)
            acc[i] = dequant_value_e4m3(codes[0][start + i], scales[0][b]);
        for (size_t r = 1; r < nranks; r++)
            for (size_t i = 0; i < len; i++)
                acc[i] = acc[i] + dequant_value_e4m3(codes[r][start + i], scales[r][b]);
        if (!all_finite(acc, len)) {
            free(acc);
            return ORACLE_NONFINITE;
        }
        quantize_one_block_e4m3(acc, len, codes_out + start, scales_out + b);
    }
    free(acc);
    return ORACLE_OK;
}

/* One ring step with E4M3 codes: dequantize, add the local values, quantize. */
int oracle_ring_step_e4m3(const uint8_t* codes_in, const float* scales_in,
                          const void* local, int dtype, size_t n, size_t block,
                          uint8_t* codes_out, float* scales_out)
{
    if (block == 0 || (dtype != ORACLE_BF16 && dtype != ORACLE_F32))
        return ORACLE_BAD_ARG;
    if (n == 0)
        return ORACLE_OK;
    for (size_t i = 0; i < n; i++)
        if (!isfinite(load_element(local, dtype, i)))
            return ORACLE_NONFINITE;
    float* acc = malloc(block * sizeof *acc);
    if (!acc)
        return ORACLE_BAD_ARG;
    size_t nb = block_count(n, block);
    for (size_t b = 0; b < nb; b++) {
        size_t start = b * block;
        size_t len = (n - start < block) ? n - start : block;
        for (size_t i = 0; i < len; i++)
            acc[i] = dequant_value_e4m3(codes_in[start + i], scales_in[b]) +
                     load_element(local, dtype, start + i);
        if (!all_finite(acc, len)) {
            free(acc);
            return ORACLE_NONFINITE;
        }
        quantize_one_block_e4m3(acc, len, codes_out + start, scales_out + b);
    }
    free(acc);
    return ORACLE_OK;
}

/* The E4M3 encoding and decoding on their own, so that tests can pin them
 * to a library conversion.  encode expects |in[i]| <= 448. */
void oracle_e4m3_encode(const float* in, size_t n, uint8_t* out)
{
    for (size_t i = 0; i < n; i++)
        out[i] = e4m3_nearest(in[i]);
}

void oracle_e4m3_decode(const uint8_t* in, size_t n, float* out)
{
    for (size_t i = 0; i < n; i++)
        out[i] = e4m3_value(in[i]);
}

/* ------------------------------------------------------------------------
 * 4-bit integer codes.  The pages name 4-bit communication quantization only
 * through the titles of later work in their reference lists ("SDP4Bit:
 * Toward 4-bit Communication Quantization in Sharded Data Parallelism ...",
 * "Echo: Error-Compensated 4-Bit Tensor-Parallel Communication ..."); no
 * format is described.  The reading here is the int8 method at 4 bits:
 *   scale  s   = fl32(absmax / 7)
 *   code   q_i = 0 if s == 0, else clamp(rne(fl32(x_i / s)), -7, 7)
 *   value  y_i = fl32((float)q_i * s)
 *   reduce and ring: as for int8 codes, with this quantizer and value.
 * Storage: two codes per byte, two's complement nibbles, element 2k in the
 * low nibble of byte k and element 2k+1 in the high nibble (by element index,
 * whatever the block length); a buffer of n elements takes ceil(n/2) bytes.
 * ------------------------------------------------------------------------ */

static int nibble_get(const uint8_t* p, size_t i)
{
    unsigned v = (p[i / 2] >> (4 * (i % 2))) & 0xFu;
    return v >= 8 ? (int)v - 16 : (int)v;
}

static void nibble_set(uint8_t* p, size_t i, int q)
{
    unsigned shift = 4 * (unsigned)(i % 2);
    p[i / 2] = (uint8_t)((p[i / 2] & ~(0xFu << shift)) | (((unsigned)q & 0xFu) << shift));
}

/* codes of one block starting at element `start` of the packed buffer */
static void quantize_one_block_int4(const float* v, size_t len, uint8_t* packed, size_t start, float* scale)
{
    float absmax = 0.0f;
    for (size_t i = 0; i < len; i++) {
        float m = fabsf(v[i]);
        if (m > absmax)
            absmax = m;
    }
    float s = absmax / 7.0f;
    *scale = s;
    for (size_t i = 0; i < len; i++) {
        if (s == 0.0f) {
            nibble_set(packed, start + i, 0);
            continue;
        }
        float t = v[i] / s;
        float r = nearbyintf(t); /* to nearest, ties to even */
        if (r > 7.0f)
            r = 7.0f;
        if (r < -7.0f)
            r = -7.0f;
        nibble_set(packed, start + i, (int)r);
    }
}

static float dequant_value_int4(const uint8_t* packed, size_t i, float s)
{
    return (float)nibble_get(packed, i) * s;
}

int oracle_quantize_int4(const void* x, int dtype, size_t n, size_t block, uint8_t* codes, float* scales)
{
    if (block == 0 || (dtype != ORACLE_BF16 && dtype != ORACLE_F32))
        return ORACLE_BAD_ARG;
    if (n == 0)
        return ORACLE_OK;
    if (!x || !codes || !scales)
        return ORACLE_BAD_ARG;
    for (size_t i = 0; i < n; i++)
        if (!isfinite(load_element(x, dtype, i)))
            return ORACLE_NONFINITE;
    float* v = malloc(block * sizeof *v);
    if (!v)
        return ORACLE_BAD_ARG;
    memset(codes, 0, (n + 1) / 2);
    size_t nb = block_count(n, block);
    for (size_t b = 0; b < nb; b++) {
        size_t start = b * block;
        size_t len = (n - start < block) ? n - start : block;
        for (size_t i = 0; i < len; i++)
            v[i] = load_element(x, dtype, start + i);
        quantize_one_block_int4(v, len, codes, start, scales + b);
    }
    free(v);
    return ORACLE_OK;
}

int oracle_dequantize_int4(const uint8_t* codes, const float* scales, size_t n, size_t block,
                           int out_dtype, void* out)
{
    if (block == 0 || (out_dtype != ORACLE_BF16 && out_dtype != ORACLE_F32))
        return ORACLE_BAD_ARG;
    for (size_t i = 0; i < n; i++) {
        float y = dequant_value_int4(codes, i, scales[i / block]);
        if (out_dtype == ORACLE_BF16)
            ((uint16_t*)out)[i] = float_to_bf16_bits(y);
        else
            ((float*)out)[i] = y;
    }
    return ORACLE_OK;
}

int oracle_reduce_int4(const uint8_t* const* codes, const float* const* scales, size_t nranks, size_t n,
                       size_t block, uint8_t* codes_out, float* scales_out)
{
    if (block == 0 || nranks == 0)
        return ORACLE_BAD_ARG;
    if (n == 0)
        return ORACLE_OK;
    float* acc = malloc(block * sizeof *acc);
    if (!acc)
        return ORACLE_BAD_ARG;
    memset(codes_out, 0, (n + 1) / 2);
    size_t nb = block_count(n, block);
    for (size_t b = 0; b < nb; b++) {
        size_t start = b * block;
        size_t len = (n - start < block) ? n - start : block;
        for (size_t i = 0; i < len; i++)
            acc[i] = dequant_value_int4(codes[0], start + i, scales[0][b]);
        for (size_t r = 1; r < nranks; r++)
            for (size_t i = 0; i < len; i++)
                acc[i] = acc[i] + dequant_value_int4(codes[r], start + i, scales[r][b]);
        if (!all_finite(acc, len)) {
            free(acc);
            return ORACLE_NONFINITE;
        }
        quantize_one_block_int4(acc, len, codes_out, start, scales_out + b);
    }
    free(acc);
    return ORACLE_OK;
}

int oracle_ring_step_int4(const uint8_t* codes_in, const float* scales_in, const void* local, int dtype,
                          size_t n, size_t block, uint8_t* codes_out, float* scales_out)
{
    if (block == 0 || (dtype != ORACLE_BF16 && dtype != ORACLE_F32))
        return ORACLE_BAD_ARG;
    if (n == 0)
        return ORACLE_OK;
    for (size_t i = 0; i < n; i++)
        if (!isfinite(load_element(local, dtype, i)))
            return ORACLE_NONFINITE;
    float* acc = malloc(block * sizeof *acc);
    if (!acc)
        return ORACLE_BAD_ARG;
    size_t nb = block_count(n, block);
    /* codes_out may not alias codes_in here: the nibbles are rewritten */
    for (size_t b = 0; b < nb; b++) {
        size_t start = b * block;
        size_t len = (n - start < block) ? n - start : block;
        for (size_t i = 0; i < len; i++)
            acc[i] = dequant_value_int4(codes_in, start + i, scales_in[b]) + load_element(local, dtype, start + i);
        if (!all_finite(acc, len)) {
            free(acc);
            return ORACLE_NONFINITE;
        }
        quantize_one_block_int4(acc, len, codes_out, start, scales_out + b);
    }
    free(acc);
    return ORACLE_OK;
}
