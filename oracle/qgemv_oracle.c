/*
 * qgemv_oracle.c -- plain, slow CPU oracle for the W4A8 block-quantized GEMV.
 *
 * TEST INFRASTRUCTURE ONLY (see qgemv_oracle.h).  Written for a reader who
 * checks it against the definitions by eye: no blocking, no fusion, no SIMD,
 * one loop per step of the definition.  Build with
 *   gcc -O2 -fno-fast-math -ffp-contract=off -std=c99
 * so that float arithmetic is plain IEEE binary32/binary64 (x86-64 SSE).
 */
#include "qgemv_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* IEEE binary16                                                            */
/* ------------------------------------------------------------------------ */

/* Exact value of a binary16 bit pattern: 1 sign bit, 5 exponent bits (bias
 * 15), 10 fraction bits; exponent 0 encodes subnormals fraction * 2^-24. */
double orc_fp16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + f), e - 25);
    }
    return sign ? -v : v;
}

/* binary32 -> binary16, round to nearest, ties to even, subnormals kept,
 * overflow to infinity.  The float is exact in double; scaling by a power of
 * two is exact; nearbyint() under the default rounding mode is ties-to-even. */
uint16_t orc_f32_to_fp16(float f) {
    double v = (double)f;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(a)) return (uint16_t)(sign | 0x7e00);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00); /* rounds past 65504 */
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: units of 2^-24; n == 1024 is the smallest normal,
         * whose encoding is exactly 1024 as well */
        double n = nearbyint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)n);
    }
    int e2;
    frexp(a, &e2);            /* a = m * 2^e2, m in [0.5, 1) */
    int e = e2 - 1;           /* a in [2^e, 2^(e+1)) */
    double n = nearbyint(ldexp(a, 10 - e)); /* in [1024, 2048] */
    if (n == 2048.0) { n = 1024.0; e += 1; }
    if (e > 15) return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(n - 1024.0));
}

void orc_fp16_to_f64_n(const uint16_t* h, int64_t n, double* out) {
    for (int64_t i = 0; i < n; i++) out[i] = orc_fp16_to_f64(h[i]);
}

void orc_f32_to_fp16_n(const float* f, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = orc_f32_to_fp16(f[i]);
}

static int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

/* ------------------------------------------------------------------------ */
/* Activation quantisation                                                  */
/* ------------------------------------------------------------------------ */

/* One block of 32 values (the W4A8 activation of "Backends and hardware",
 * section "CPU"):
 *   amax = max |x_i|
 *   amax == 0: d = 0, q_i = 0, s = 0
 *   else:      d = amax / 127 (binary32 division),
 *              q_i = clamp(round_half_away(x_i / d), -127, 127) with a binary32
 *              division, d stored as binary16 (RNE), s = sum q_i. */
static void quantize_block(const float* x, int n_valid, int8_t q[32],
                           uint16_t* d, int32_t* s) {
    float amax = 0.0f;
    for (int i = 0; i < n_valid; i++) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        for (int i = 0; i < 32; i++) q[i] = 0;
        *d = 0;
        *s = 0;
        return;
    }
    float d32 = amax / 127.0f;
    int32_t sum = 0;
    for (int i = 0; i < 32; i++) {
        int32_t qi = 0;
        if (i < n_valid) {
            float r = roundf(x[i] / d32);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            qi = (int32_t)r;
        }
        q[i] = (int8_t)qi;
        sum += qi;
    }
    *d = orc_f32_to_fp16(d32);
    *s = sum;
}

void orc_quantize_act(const float* x, int64_t M, int64_t K, int64_t ldx,
                      int8_t* q, uint16_t* d, int32_t* s) {
    int64_t Kp = round_up(K, 256);
    int64_t nb = Kp / 32;
    for (int64_t m = 0; m < M; m++) {
        for (int64_t b = 0; b < nb; b++) {
            int64_t k0 = 32 * b;
            int n_valid = (k0 >= K) ? 0 : (int)((K - k0) < 32 ? (K - k0) : 32);
            quantize_block(x + m * ldx + k0, n_valid, q + m * Kp + k0,
                           d + m * nb + b, s + m * nb + b);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Block layouts (GGUF convention, little-endian fields)                    */
/* ------------------------------------------------------------------------ */

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Q4_0, 18 bytes per 32 weights: fp16 d, then 16 bytes; byte j holds element
 * j in its low nibble and element j+16 in its high nibble.  w = d*(code-8). */
void orc_unpack_q4_0(const uint8_t* blk, uint8_t codes[32], uint16_t* d) {
    *d = rd16(blk);
    for (int j = 0; j < 16; j++) {
        codes[j] = blk[2 + j] & 0x0f;
        codes[j + 16] = blk[2 + j] >> 4;
    }
}

/* Q4_K, 144 bytes per 256 weights: fp16 d, fp16 dmin, 12 bytes of 6-bit
 * scales and mins for the 8 sub-blocks of 32, then 128 bytes of nibbles.
 *   sub-block j < 4 : scale = b[j] & 63,           min = b[j+4] & 63
 *   sub-block j >= 4: scale = (b[j+4] & 15) | ((b[j-4] >> 6) << 4)
 *                     min   = (b[j+4] >> 4) | ((b[j]   >> 6) << 4)
 * Nibbles: chunk c = 0..3 covers 64 weights; byte qs[32c + l] holds element
 * 64c + l (low nibble, sub-block 2c) and 64c + 32 + l (high, sub-block 2c+1).
 * w = d*scale_j*code - dmin*min_j. */
void orc_unpack_q4_k(const uint8_t* sb, uint8_t codes[256], uint8_t sc[8],
                     uint8_t mn[8], uint16_t* d, uint16_t* dmin) {
    const uint8_t* b = sb + 4;
    const uint8_t* qs = sb + 16;
    *d = rd16(sb);
    *dmin = rd16(sb + 2);
    for (int j = 0; j < 4; j++) {
        sc[j] = b[j] & 63;
        mn[j] = b[j + 4] & 63;
    }
    for (int j = 4; j < 8; j++) {
        sc[j] = (uint8_t)((b[j + 4] & 15) | ((b[j - 4] >> 6) << 4));
        mn[j] = (uint8_t)((b[j + 4] >> 4) | ((b[j] >> 6) << 4));
    }
    for (int c = 0; c < 4; c++) {
        for (int l = 0; l < 32; l++) {
            codes[64 * c + l] = qs[32 * c + l] & 0x0f;
            codes[64 * c + 32 + l] = qs[32 * c + l] >> 4;
        }
    }
}

/* Q6_K, 210 bytes per 256 weights: ql[128] (low 4 bits), qh[64] (high 2 bits),
 * 16 int8 scales (one per 16 weights), fp16 d.  For half h = 0, 1 and
 * l = 0..31, with L = ql + 64h, H = qh + 32h, e = 128h:
 *   element e+l    : low nibble of L[l],    high bits = bits 0-1 of H[l]
 *   element e+l+32 : low nibble of L[l+32], high bits = bits 2-3 of H[l]
 *   element e+l+64 : high nibble of L[l],   high bits = bits 4-5 of H[l]
 *   element e+l+96 : high nibble of L[l+32],high bits = bits 6-7 of H[l]
 * code = low | high << 4 (0..63); element i uses scale sc[i/16];
 * w = d*sc*(code-32). */
void orc_unpack_q6_k(const uint8_t* sb, uint8_t codes[256], int8_t sc[16],
                     uint16_t* d) {
    const uint8_t* ql = sb;
    const uint8_t* qh = sb + 128;
    for (int i = 0; i < 16; i++) sc[i] = (int8_t)sb[192 + i];
    *d = rd16(sb + 208);
    for (int h = 0; h < 2; h++) {
        const uint8_t* L = ql + 64 * h;
        const uint8_t* H = qh + 32 * h;
        int e = 128 * h;
        for (int l = 0; l < 32; l++) {
            codes[e + l]      = (uint8_t)((L[l] & 0x0f)      | (((H[l] >> 0) & 3) << 4));
            codes[e + l + 32] = (uint8_t)((L[l + 32] & 0x0f) | (((H[l] >> 2) & 3) << 4));
            codes[e + l + 64] = (uint8_t)((L[l] >> 4)        | (((H[l] >> 4) & 3) << 4));
            codes[e + l + 96] = (uint8_t)((L[l + 32] >> 4)   | (((H[l] >> 6) & 3) << 4));
        }
    }
}

/* Q8_0, 34 bytes per 32 weights: fp16 d, then 32 int8 codes.  w = d*code. */
void orc_unpack_q8_0(const uint8_t* blk, int8_t codes[32], uint16_t* d) {
    *d = rd16(blk);
    for (int j = 0; j < 32; j++) codes[j] = (int8_t)blk[2 + j];
}

int64_t orc_row_bytes(int fmt, int64_t K) {
    switch (fmt) {
    case ORC_Q4_0: return (K / 32) * 18;
    case ORC_Q4_K: return (round_up(K, 256) / 256) * 144;
    case ORC_Q6_K: return (round_up(K, 256) / 256) * 210;
    case ORC_Q8_0: return (K / 32) * 34;
    default: return -1;
    }
}

int64_t orc_nblk(int fmt, int64_t K) {
    switch (fmt) {
    case ORC_Q4_0: return K / 32;
    case ORC_Q4_K: return round_up(K, 256) / 32;
    case ORC_Q6_K: return round_up(K, 256) / 16;
    case ORC_Q8_0: return K / 32;
    default: return -1;
    }
}

/* ------------------------------------------------------------------------ */
/* Integer block dots                                                       */
/* ------------------------------------------------------------------------ */

/* Q4_0 block b: D = sum_{i<32} (code_i - 8) * q_i
 * Q4_K sub-block j of super-block S: D = sum_{i<32} code_i * q_i (codes 0..15;
 *      the min is applied through the activation block sum)
 * Q6_K group g of super-block S: D16 = sum_{i<16} (code_i - 32) * q_i
 * Q8_0 block b: D = sum_{i<32} code_i * q_i */
static void row_block_dots(int fmt, const uint8_t* row, int64_t K,
                           const int8_t* q, int32_t* dots) {
    int64_t Kp = round_up(K, 256);
    if (fmt == ORC_Q4_0) {
        for (int64_t b = 0; b < K / 32; b++) {
            uint8_t codes[32];
            uint16_t d;
            orc_unpack_q4_0(row + 18 * b, codes, &d);
            int32_t D = 0;
            for (int i = 0; i < 32; i++) D += ((int32_t)codes[i] - 8) * q[32 * b + i];
            dots[b] = D;
        }
    } else if (fmt == ORC_Q8_0) {
        for (int64_t b = 0; b < K / 32; b++) {
            int8_t codes[32];
            uint16_t d;
            orc_unpack_q8_0(row + 34 * b, codes, &d);
            int32_t D = 0;
            for (int i = 0; i < 32; i++) D += (int32_t)codes[i] * q[32 * b + i];
            dots[b] = D;
        }
    } else if (fmt == ORC_Q4_K) {
        for (int64_t S = 0; S < Kp / 256; S++) {
            uint8_t codes[256], sc[8], mn[8];
            uint16_t d, dmin;
            orc_unpack_q4_k(row + 144 * S, codes, sc, mn, &d, &dmin);
            for (int j = 0; j < 8; j++) {
                int32_t D = 0;
                for (int i = 0; i < 32; i++)
                    D += (int32_t)codes[32 * j + i] * q[256 * S + 32 * j + i];
                dots[8 * S + j] = D;
            }
        }
    } else if (fmt == ORC_Q6_K) {
        for (int64_t S = 0; S < Kp / 256; S++) {
            uint8_t codes[256];
            int8_t sc[16];
            uint16_t d;
            orc_unpack_q6_k(row + 210 * S, codes, sc, &d);
            for (int g = 0; g < 16; g++) {
                int32_t D = 0;
                for (int i = 0; i < 16; i++)
                    D += ((int32_t)codes[16 * g + i] - 32) * q[256 * S + 16 * g + i];
                dots[16 * S + g] = D;
            }
        }
    }
}

void orc_block_dots(int fmt, const uint8_t* w, int64_t N, int64_t K,
                    int64_t row0, int64_t nrows, const int8_t* q,
                    int32_t* dots) {
    (void)N;
    int64_t rb = orc_row_bytes(fmt, K);
    int64_t nblk = orc_nblk(fmt, K);
    for (int64_t r = 0; r < nrows; r++)
        row_block_dots(fmt, w + (row0 + r) * rb, K, q, dots + r * nblk);
}

/* ------------------------------------------------------------------------ */
/* Row outputs                                                              */
/* ------------------------------------------------------------------------ */

/* One row against one activation row, in float64 (f() = exact fp16 value):
 *   Q4_0: y = sum_b f(dw_b) f(dx_b) D_b
 *   Q8_0: y = sum_b f(dw_b) f(dx_b) D_b
 *   Q4_K: y = sum_S sum_j [ f(d_S) sc_Sj f(dx_b) D_Sj - f(dmin_S) m_Sj f(dx_b) s_b ],
 *         b = 8S + j, over the sub-blocks that start below K
 *   Q6_K: y = sum_S sum_g f(d_S) sc_Sg f(dx_b) D16_Sg, b = 8S + g/2,
 *         over the groups that start below K
 * Every product above is exact in float64 (at most 11+11+7+17 significant
 * bits); T collects |each term|, the Q4_K scale and min terms separately. */
static void row_output(int fmt, const uint8_t* row, int64_t K,
                       const int8_t* q, const uint16_t* dx, const int32_t* s,
                       double* y_out, double* T_out) {
    int64_t Kp = round_up(K, 256);
    int64_t nblk = orc_nblk(fmt, K);
    int32_t* dots = (int32_t*)malloc((size_t)nblk * sizeof(int32_t));
    row_block_dots(fmt, row, K, q, dots);
    double y = 0.0, T = 0.0;
    if (fmt == ORC_Q4_0 || fmt == ORC_Q8_0) {
        int64_t bb = (fmt == ORC_Q4_0) ? 18 : 34;
        for (int64_t b = 0; b < K / 32; b++) {
            double t = orc_fp16_to_f64(rd16(row + bb * b)) *
                       orc_fp16_to_f64(dx[b]) * (double)dots[b];
            y += t;
            T += fabs(t);
        }
    } else if (fmt == ORC_Q4_K) {
        for (int64_t S = 0; S < Kp / 256; S++) {
            uint8_t codes[256], sc[8], mn[8];
            uint16_t d, dmin;
            orc_unpack_q4_k(row + 144 * S, codes, sc, mn, &d, &dmin);
            for (int j = 0; j < 8; j++) {
                int64_t b = 8 * S + j;
                if (32 * b >= K) break;
                double fdx = orc_fp16_to_f64(dx[b]);
                double t1 = orc_fp16_to_f64(d) * (double)sc[j] * fdx * (double)dots[b];
                double t2 = orc_fp16_to_f64(dmin) * (double)mn[j] * fdx * (double)s[b];
                y += t1 - t2;
                T += fabs(t1) + fabs(t2);
            }
        }
    } else if (fmt == ORC_Q6_K) {
        for (int64_t S = 0; S < Kp / 256; S++) {
            uint8_t codes[256];
            int8_t sc[16];
            uint16_t d;
            orc_unpack_q6_k(row + 210 * S, codes, sc, &d);
            for (int g = 0; g < 16; g++) {
                int64_t e = 256 * S + 16 * g;
                if (e >= K) break;
                int64_t b = 8 * S + g / 2;
                double t = orc_fp16_to_f64(d) * (double)sc[g] *
                           orc_fp16_to_f64(dx[b]) * (double)dots[16 * S + g];
                y += t;
                T += fabs(t);
            }
        }
    }
    free(dots);
    *y_out = y;
    *T_out = T;
}

void orc_gemv(int fmt, const uint8_t* w, int64_t N, int64_t K,
              int64_t row0, int64_t nrows,
              const int8_t* q, const uint16_t* d, const int32_t* s,
              double* y, double* T) {
    (void)N;
    int64_t rb = orc_row_bytes(fmt, K);
    for (int64_t r = 0; r < nrows; r++)
        row_output(fmt, w + (row0 + r) * rb, K, q, d, s, y + r, T + r);
}

/* "C = A x B is row-independent" (colibri GPU backends, eligibility gates):
 * activation row m against the weights is exactly the single-row product. */
void orc_gemm(int fmt, const uint8_t* w, int64_t N, int64_t K, int64_t M,
              int64_t row0, int64_t nrows,
              const int8_t* q, const uint16_t* d, const int32_t* s,
              double* y, double* T) {
    int64_t Kp = round_up(K, 256);
    int64_t nb = Kp / 32;
    for (int64_t m = 0; m < M; m++)
        orc_gemv(fmt, w, N, K, row0, nrows, q + m * Kp, d + m * nb, s + m * nb,
                 y + m * nrows, T + m * nrows);
}

/* SwiGLU (llambda.lisp README, supported architectures; VKNN guide): the FFN
 * hidden state is SiLU(gate) * up with SiLU(g) = g / (1 + e^-g). */
void orc_silu_mul(const float* gu, int64_t N, double* h) {
    for (int64_t i = 0; i < N; i++) {
        double g = (double)gu[i];
        double u = (double)gu[N + i];
        h[i] = g / (1.0 + exp(-g)) * u;
    }
}
