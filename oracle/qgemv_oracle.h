/*
 * qgemv_oracle.h -- plain, slow CPU oracle for the W4A8 block-quantized GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may call into this code.  The product library
 * (libqgemv) neither links nor includes it, and it shares no source, header,
 * table or helper with the GPU path.
 *
 * What it computes (each function below names the passage it follows):
 *   - "Backends and hardware" (llamay docs), section "CPU": the activation is
 *     quantised to int8 once per matmul and the weight rows are never
 *     materialised; the inner product is an integer (W4A8) dot product
 *     (section "CUDA" names the 4 x int8 dot as that inner product).
 *   - "Running an LLM on VKNN", section 7 "Precision": accumulation across
 *     blocks is floating point regardless of the storage tier.
 *   - Block layouts: the GGUF convention for Q4_0 / Q4_K / Q6_K / Q8_0 (the
 *     llambda.lisp README reads Q4_K_M and Q6_K tensors straight from .gguf
 *     files, "Features & Architecture").  The byte-level arrangement is a
 *     reading, not something the pages print; it is spelled out next to each
 *     unpack routine.
 *
 * Arithmetic: integers are exact; every floating-point row output is summed in
 * float64 from exactly representable per-block terms, so the only rounding is
 * the float64 summation itself (relative error ~1e-16 of sum|terms|).
 *
 * Format ids: 0 = Q4_0, 1 = Q4_K, 2 = Q6_K, 3 = Q8_0.
 * All pointers are host pointers.  K must be a positive multiple of 32.
 * Kp = K rounded up to 256 (the activation row length and the padded K-quant
 * row length); for Q4_0 and Q8_0 rows hold exactly K/32 blocks.
 */
#ifndef QGEMV_ORACLE_H
#define QGEMV_ORACLE_H
#include <stdint.h>

#define ORC_Q4_0 0
#define ORC_Q4_K 1
#define ORC_Q6_K 2
#define ORC_Q8_0 3

/* IEEE binary16 helpers (own implementation, exact decode, RNE encode). */
double   orc_fp16_to_f64(uint16_t h);
uint16_t orc_f32_to_fp16(float f);
void     orc_fp16_to_f64_n(const uint16_t* h, int64_t n, double* out);
void     orc_f32_to_fp16_n(const float* f, int64_t n, uint16_t* out);

/* Activation quantisation, one row-major fp32 matrix x[M][ldx] with K valid
 * columns -> q int8 [M][Kp], d fp16 bits [M][Kp/32], s int32 [M][Kp/32].
 * Blocks past K are all zero. */
void orc_quantize_act(const float* x, int64_t M, int64_t K, int64_t ldx,
                      int8_t* q, uint16_t* d, int32_t* s);

/* Unpack one block / super-block into plain integer codes and scale fields. */
void orc_unpack_q4_0(const uint8_t* blk, uint8_t codes[32], uint16_t* d);
void orc_unpack_q4_k(const uint8_t* sb, uint8_t codes[256], uint8_t sc[8],
                     uint8_t mn[8], uint16_t* d, uint16_t* dmin);
void orc_unpack_q6_k(const uint8_t* sb, uint8_t codes[256], int8_t sc[16],
                     uint16_t* d);
void orc_unpack_q8_0(const uint8_t* blk, int8_t codes[32], uint16_t* d);

/* Bytes per stored weight row. */
int64_t orc_row_bytes(int fmt, int64_t K);

/* Per-block int32 dots of rows [row0, row0+nrows) against activation codes
 * q (one activation row, length Kp).  dots is [nrows][nblk] with
 * nblk = K/32 (Q4_0, Q8_0), Kp/32 (Q4_K), Kp/16 (Q6_K). */
int64_t orc_nblk(int fmt, int64_t K);
void orc_block_dots(int fmt, const uint8_t* w, int64_t N, int64_t K,
                    int64_t row0, int64_t nrows, const int8_t* q,
                    int32_t* dots);

/* Row outputs for rows [row0, row0+nrows) against one activation row:
 * y[i] = the definition summed in float64, T[i] = sum of |every fp term|. */
void orc_gemv(int fmt, const uint8_t* w, int64_t N, int64_t K,
              int64_t row0, int64_t nrows,
              const int8_t* q, const uint16_t* d, const int32_t* s,
              double* y, double* T);

/* M activation rows against the same weights: y[m][i], T[m][i] over
 * rows [row0, row0+nrows). Row m is exactly orc_gemv on activation row m. */
void orc_gemm(int fmt, const uint8_t* w, int64_t N, int64_t K, int64_t M,
              int64_t row0, int64_t nrows,
              const int8_t* q, const uint16_t* d, const int32_t* s,
              double* y, double* T);

/* SwiGLU glue: gu = [gate (N) | up (N)] fp32 -> h[i] = silu(g_i) * u_i in
 * float64 with silu(g) = g / (1 + exp(-g)). */
void orc_silu_mul(const float* gu, int64_t N, double* h);

#endif
