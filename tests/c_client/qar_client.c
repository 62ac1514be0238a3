/* A plain C99 program that runs the path on the GPU through libqar's C ABI
 * only (no Python, no torch): device buffers from hipMalloc, four ranks'
 * bf16 data quantized, the one-shot reduce with a fused bf16 output, the
 * one-kernel step with rank 1 as its own rank, a standalone fp32 dequantize
 * and a ring step; every result compared bit for bit with the CPU oracle
 * (oracle/qar_oracle.c, linked as test infrastructure).  Prints "ok" and
 * exits 0 when everything matches. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "qar.h"

/* the oracle's entry points (oracle/qar_oracle.c) */
int oracle_quantize(const void* x, int dtype, size_t n, size_t block, int8_t* codes, float* scales);
int oracle_dequantize_f32(const int8_t* codes, const float* scales, size_t n, size_t block, float* out);
int oracle_dequantize_bf16(const int8_t* codes, const float* scales, size_t n, size_t block, uint16_t* out);
int oracle_reduce(const int8_t* const* codes, const float* const* scales, size_t nranks, size_t n, size_t block,
                  int8_t* codes_out, float* scales_out);
int oracle_ring_step(const int8_t* codes_in, const float* scales_in, const void* local, int dtype, size_t n,
                     size_t block, int8_t* codes_out, float* scales_out);

enum { N = 4, BLOCK = 128, NELEM = 3 * 4096 + 5 * BLOCK, NB = NELEM / BLOCK };

static int failures = 0;

#define HIP_CHECK(call)                                                                             \
    do {                                                                                            \
        hipError_t e_ = (call);                                                                     \
        if (e_ != hipSuccess) {                                                                     \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_));              \
            exit(3);                                                                                \
        }                                                                                           \
    } while (0)

#define QAR_CHECK(call)                                                                             \
    do {                                                                                            \
        qar_status s_ = (call);                                                                     \
        if (s_ != QAR_OK) {                                                                         \
            fprintf(stderr, "%s:%d: %s %s\n", __FILE__, __LINE__, qar_status_string(s_), qar_last_error()); \
            exit(4);                                                                                \
        }                                                                                           \
    } while (0)

static void same(const void* got, const void* want, size_t bytes, const char* what) {
    if (memcmp(got, want, bytes) != 0) {
        const unsigned char* g = got;
        const unsigned char* w = want;
        size_t i = 0;
        while (g[i] == w[i]) ++i;
        fprintf(stderr, "%s: first difference at byte %zu\n", what, i);
        ++failures;
    }
}

/* bf16 patterns with exponents over a wide range, both signs (xorshift32) */
static void fill_bf16(uint16_t* x, size_t n, uint32_t seed) {
    uint32_t s = seed * 2654435761u + 1u;
    for (size_t i = 0; i < n; ++i) {
        s ^= s << 13;
        s ^= s >> 17;
        s ^= s << 5;
        const uint32_t exponent = 100u + (s >> 8) % 48u;   /* 2^-27 .. 2^20 */
        x[i] = (uint16_t)(((s >> 31) << 15) | (exponent << 7) | (s & 0x7Fu));
    }
}

int main(void) {
    uint16_t* x[N];
    int8_t* codes[N];
    float* scales[N];
    uint16_t* d_x[N];
    int8_t* d_codes[N];
    float* d_scales[N];
    for (int r = 0; r < N; ++r) {
        x[r] = malloc(NELEM * sizeof(uint16_t));
        codes[r] = malloc(NELEM);
        scales[r] = malloc(NB * sizeof(float));
        fill_bf16(x[r], NELEM, 11u + (uint32_t)r);
        HIP_CHECK(hipMalloc((void**)&d_x[r], NELEM * sizeof(uint16_t)));
        HIP_CHECK(hipMalloc((void**)&d_codes[r], NELEM));
        HIP_CHECK(hipMalloc((void**)&d_scales[r], NB * sizeof(float)));
        HIP_CHECK(hipMemcpy(d_x[r], x[r], NELEM * sizeof(uint16_t), hipMemcpyHostToDevice));
    }
    int8_t *d_rc, *d_sc, *d_ringc;
    float *d_rs, *d_ss, *d_y, *d_rings;
    uint16_t *d_out, *d_sout;
    HIP_CHECK(hipMalloc((void**)&d_rc, NELEM));
    HIP_CHECK(hipMalloc((void**)&d_sc, NELEM));
    HIP_CHECK(hipMalloc((void**)&d_ringc, NELEM));
    HIP_CHECK(hipMalloc((void**)&d_rs, NB * sizeof(float)));
    HIP_CHECK(hipMalloc((void**)&d_ss, NB * sizeof(float)));
    HIP_CHECK(hipMalloc((void**)&d_rings, NB * sizeof(float)));
    HIP_CHECK(hipMalloc((void**)&d_y, NELEM * sizeof(float)));
    HIP_CHECK(hipMalloc((void**)&d_out, NELEM * sizeof(uint16_t)));
    HIP_CHECK(hipMalloc((void**)&d_sout, NELEM * sizeof(uint16_t)));
    hipStream_t st;
    HIP_CHECK(hipStreamCreate(&st));

    for (int r = 0; r < N; ++r)
        QAR_CHECK(qar_quantize_blocks(d_x[r], QAR_BF16, NELEM, BLOCK, d_codes[r], d_scales[r], st));
    QAR_CHECK(qar_reduce_quantized((const int8_t* const*)d_codes, (const float* const*)d_scales, N, NELEM, BLOCK,
                                   d_rc, d_rs, d_out, QAR_BF16, st));
    QAR_CHECK(qar_dequantize(d_rc, d_rs, NELEM, BLOCK, d_y, QAR_F32, st));
    QAR_CHECK(qar_ring_step(d_codes[0], d_scales[0], d_x[1], QAR_BF16, NELEM, BLOCK, d_ringc, d_rings, st));
    /* the one-kernel step, rank 1 quantized again from its input */
    QAR_CHECK(qar_quantize_reduce(d_x[1], QAR_BF16, 1, d_codes, d_scales, N, NELEM, BLOCK, d_sc, d_ss, d_sout,
                                  QAR_BF16, st));
    HIP_CHECK(hipStreamSynchronize(st));

    /* the oracle */
    for (int r = 0; r < N; ++r)
        if (oracle_quantize(x[r], 0, NELEM, BLOCK, codes[r], scales[r]) != 0) return 5;
    int8_t* rc = malloc(NELEM);
    float* rs = malloc(NB * sizeof(float));
    uint16_t* out = malloc(NELEM * sizeof(uint16_t));
    float* y = malloc(NELEM * sizeof(float));
    int8_t* ringc = malloc(NELEM);
    float* rings = malloc(NB * sizeof(float));
    if (oracle_reduce((const int8_t* const*)codes, (const float* const*)scales, N, NELEM, BLOCK, rc, rs) != 0)
        return 5;
    oracle_dequantize_bf16(rc, rs, NELEM, BLOCK, out);
    oracle_dequantize_f32(rc, rs, NELEM, BLOCK, y);
    if (oracle_ring_step(codes[0], scales[0], x[1], 0, NELEM, BLOCK, ringc, rings) != 0) return 5;

    /* compare */
    int8_t* g8 = malloc(NELEM);
    float* gs = malloc(NB * sizeof(float));
    uint16_t* g16 = malloc(NELEM * sizeof(uint16_t));
    float* g32 = malloc(NELEM * sizeof(float));
    for (int r = 0; r < N; ++r) {
        HIP_CHECK(hipMemcpy(g8, d_codes[r], NELEM, hipMemcpyDeviceToHost));
        HIP_CHECK(hipMemcpy(gs, d_scales[r], NB * sizeof(float), hipMemcpyDeviceToHost));
        same(g8, codes[r], NELEM, "rank codes");
        same(gs, scales[r], NB * sizeof(float), "rank scales");
    }
    HIP_CHECK(hipMemcpy(g8, d_rc, NELEM, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(gs, d_rs, NB * sizeof(float), hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(g16, d_out, NELEM * sizeof(uint16_t), hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(g32, d_y, NELEM * sizeof(float), hipMemcpyDeviceToHost));
    same(g8, rc, NELEM, "reduce codes");
    same(gs, rs, NB * sizeof(float), "reduce scales");
    same(g16, out, NELEM * sizeof(uint16_t), "reduce bf16 out");
    same(g32, y, NELEM * sizeof(float), "dequantize fp32");
    HIP_CHECK(hipMemcpy(g8, d_sc, NELEM, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(gs, d_ss, NB * sizeof(float), hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(g16, d_sout, NELEM * sizeof(uint16_t), hipMemcpyDeviceToHost));
    same(g8, rc, NELEM, "step codes");
    same(gs, rs, NB * sizeof(float), "step scales");
    same(g16, out, NELEM * sizeof(uint16_t), "step bf16 out");
    HIP_CHECK(hipMemcpy(g8, d_ringc, NELEM, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(gs, d_rings, NB * sizeof(float), hipMemcpyDeviceToHost));
    same(g8, ringc, NELEM, "ring codes");
    same(gs, rings, NB * sizeof(float), "ring scales");

    HIP_CHECK(hipStreamDestroy(st));
    if (failures) return 6;
    printf("ok\n");
    return 0;
}
