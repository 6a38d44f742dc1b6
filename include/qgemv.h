/*
 * qgemv.h -- C ABI of libqgemv: W4A8 block-quantized GEMV for AMD MI355X (gfx950).
 *
 * The operation ("Backends and hardware", llamay docs, section "CPU"): the
 * activation is quantised to int8 once per matmul, in blocks of 32 with an
 * fp16 scale and an int32 code sum, and each weight row stays in its packed
 * block format -- it is never expanded to float.  A row is multiplied block by
 * block with 4 x int8 integer dot products (section "CUDA" names that dot as
 * the W4A8 inner product), the block scales (and, for Q4_K, mins) are applied
 * in fp32, and the row is reduced.  Accumulation across blocks is fp32
 * ("Running an LLM on VKNN", section 7 "Precision").
 *
 * Generation 1.  All data pointers are DEVICE pointers (HIP global memory)
 * unless stated otherwise; sizes are element counts.
 *
 * Stored weight formats (GGUF block layouts, little-endian fields), row-major,
 * one row after another with no gap:
 *   Q4_0  18 B per 32 weights : fp16 d | 16 B, byte j = code j (low nibble),
 *                               code j+16 (high nibble); w = d*(code-8)
 *   Q4_K 144 B per 256 weights: fp16 d | fp16 dmin | 12 B of 6-bit scale and
 *                               min for 8 sub-blocks of 32 | 128 B nibbles;
 *                               w = d*scale_j*code - dmin*min_j
 *   Q6_K 210 B per 256 weights: 128 B low nibbles | 64 B high 2-bit pairs |
 *                               16 int8 scales (one per 16) | fp16 d;
 *                               w = d*scale*(code-32)
 *   Q8_0  34 B per 32 weights : fp16 d | 32 int8 codes; w = d*code
 *   Q6_K_R8: Q6_K rows rearranged at load into aligned tiles of 8
 *            super-blocks by qgemv_q6_k_repack (see there)
 * K-quant (Q4_K, Q6_K) rows hold ceil(K/256) super-blocks; the weights past K
 * in the last one must have zero codes, scales and mins.  Q4_0 / Q8_0 rows
 * hold exactly K/32 blocks.
 *
 * Activation layout (this library's, struct of arrays), Kp = K rounded up to
 * a multiple of 256:  q int8 [M][Kp], d fp16 bits [M][Kp/32], s int32
 * [M][Kp/32].  Blocks past K are all zero.
 *
 * Conventions shared by every entry point:
 *   - Argument gates run in a fixed order, cheapest first, and the first
 *     failure returns: NULL pointers, then shapes, then limits of this library,
 *     then alignment, then the device (colibri GPU backends, "Eligibility
 *     gates": every gate returns).  On any error nothing is launched and no
 *     output is written (same page, "Failure invariant": a failure is never a
 *     partial result).  qgemv_last_error() then names the reason.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream)
 *     and returns without waiting; there is no host synchronisation, no
 *     host<->device copy and no allocation, so calls can be captured into a
 *     HIP graph.  Faults inside a kernel surface at the caller's next
 *     synchronisation, as usual for HIP.
 *   - The library keeps no per-call state (only the thread-local error text
 *     and timing setting below): concurrent calls on different streams are
 *     safe as long as their output buffers do not overlap.
 *     Inputs and outputs of one call must not alias.
 *   - An empty problem (N == 0 or M == 0) returns QGEMV_OK without launching.
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QGEMV_ABI_VERSION 1

/* Largest K accepted by the GEMV and small-M entry points in this library. */
#define QGEMV_K_MAX 32768
/* Most matrices one qgemv_multi / qgemv_quantize_multi call takes. */
#define QGEMV_MULTI_MAX 8
/* Largest M accepted by qgemm_q4_k_small_m. */
#define QGEMV_M_MAX 64

typedef void* qgemv_stream_t;

/* Status codes, numbered in the order the gates run (so the limits of this
 * library, checked before alignment, come before QGEMV_E_ALIGN). */
typedef enum {
    QGEMV_OK = 0,
    QGEMV_E_NULL = 1,        /* a required pointer is NULL */
    QGEMV_E_SHAPE = 2,       /* negative size, K not a positive multiple of 32, ldx < K, ... */
    QGEMV_E_UNSUPPORTED = 3, /* valid but declined by this library (K > QGEMV_K_MAX, M > QGEMV_M_MAX, bad enum) */
    QGEMV_E_ALIGN = 4,       /* w, q not 16-byte aligned; d 2-byte; x, s, y, h, gu, dots 4-byte
                                (x 16-byte for the products that quantise it) */
    QGEMV_E_DEVICE = 5,      /* no current HIP device, or it is not gfx950 */
    QGEMV_E_LAUNCH = 6       /* the kernel launch itself failed */
} qgemv_status;

/* QGEMV_FMT_Q6_K_R8: Q6_K repacked by qgemv_q6_k_repack (see there). */
enum {
    QGEMV_FMT_Q4_0 = 0,
    QGEMV_FMT_Q4_K = 1,
    QGEMV_FMT_Q6_K = 2,
    QGEMV_FMT_Q8_0 = 3,
    QGEMV_FMT_Q6_K_R8 = 4
};
/* Small-M variants.  QGEMV_VARIANT_MFMA runs the int8 matrix cores with the
 * faster of two kernels for the format, shape and bucket of M (measured);
 * QGEMV_VARIANT_MFMA_STAGED forces the kernel that stages every K step of
 * weights and activation through LDS, QGEMV_VARIANT_MFMA_STREAM the one in
 * which every wave streams its own weight rows into registers and only the
 * activation is shared through LDS, QGEMV_VARIANT_MFMA_RESIDENT (Q4_K, M <=
 * 16, K <= 16384; elsewhere the MFMA choice) the one in which each wave
 * keeps the activation of its slice of K in registers and streams its own
 * 16-row weight tiles.  All compute the same products. */
enum {
    QGEMV_VARIANT_AUTO = 0,
    QGEMV_VARIANT_DOT4 = 1,
    QGEMV_VARIANT_MFMA = 2,
    QGEMV_VARIANT_MFMA_STAGED = 3,
    QGEMV_VARIANT_MFMA_STREAM = 4,
    QGEMV_VARIANT_MFMA_RESIDENT = 5
};

/* Returns QGEMV_ABI_VERSION of the loaded library.  A caller built against a
 * different generation must refuse the library as a whole rather than bind
 * part of it (colibri GPU backends, the XDNA helper's ABI: a helper is usable
 * only when it reports the expected ABI generation and exports every entry
 * point the host requires; binding is all-or-nothing).  No arguments, no
 * device access, never fails. */
int qgemv_abi_version(void);

/* Static, never-NULL name and one-line meaning of a status code; an unknown
 * code gives "QGEMV_E_UNKNOWN: ...".  Each refusal has its own status because
 * each has its own fix (colibri GPU backends, provisioning diagnostics: one
 * named diagnostic per kind of failure; "Backends and hardware", section
 * "CUDA": a backend declines with a message naming the reason).  The string
 * belongs to the library and must not be freed; no device access. */
const char* qgemv_status_str(int status);

/* Static string naming what this build carries: ABI generation, target
 * architecture, weight formats, kernel variants and limits ("Backends and
 * hardware", section "Environment": the version command prints the kernel
 * sets, formats and architectures a given build actually carries, the first
 * thing to check when a number looks wrong).  Owned by the library, never
 * NULL, no device access. */
const char* qgemv_build_info(void);

/* Reason for the most recent non-OK status returned to the calling thread
 * (thread-local, overwritten by the next failing call; "" if none). */
const char* qgemv_last_error(void);

/* Kernel timing, a measurement aid that no product formula needs.  Arms the
 * calling host thread so that the next kernel this library launches from
 * that thread records `start` (a hipEvent_t, or NULL) when the kernel begins
 * and `stop` (a hipEvent_t, or NULL) when it ends.  hipEventElapsedTime
 * (start, stop) is then that kernel's own duration, without the time the
 * stream spent on earlier work or between launches.  The events are created
 * and destroyed by the caller and must outlive the timed launch.  One launch
 * consumes the setting: an entry point that launches several kernels times
 * its first; a call that returns an error before launching leaves it armed.
 * qgemv_time_next_launch(NULL, NULL) disarms.  Meant for eager launches:
 * disarm before capturing a stream into a HIP graph.  Only this thread-local
 * pair is stored; returns QGEMV_OK. */
qgemv_status qgemv_time_next_launch(void* start, void* stop);

/* Measurement aid: reads `bytes` of device memory at buf once, with 16-byte
 * loads spread over the whole device (wg_per_cu workgroups of 256 threads per
 * compute unit, 1..32), and discards the data -- the plain streaming read
 * whose rate the GEMV kernels, bound by streaming their weights, are compared
 * with ("Running an LLM on VKNN", Performance: the decode step is
 * weight-memory-bandwidth-bound).  nontemporal != 0 marks the loads
 * non-temporal.  buf: 16-byte aligned, bytes a positive multiple of 16;
 * sink: device uint32, written only in the (practically impossible) case
 * that the folded data equal a fixed constant, so that no load can be
 * elided.  No allocation; gates and errors as for the GEMVs. */
qgemv_status qgemv_stream_read(const void* buf, int64_t bytes, int nontemporal,
                               uint32_t* sink, int wg_per_cu, qgemv_stream_t stream);

/* Activation quantisation ("Backends and hardware", section "CPU": quantised
 * to int8 once per matmul).  x: fp32 [M][ldx] with K valid columns
 * (K % 32 == 0, ldx >= K).  For every block of 32 values:
 *     amax = max|x_i|;  amax == 0 -> d = 0, q_i = 0, s = 0;  otherwise
 *     d32 = amax / 127 (IEEE fp32 division),
 *     q_i = clamp(round_half_away(x_i / d32), -127, 127) (IEEE division),
 *     d = fp16(d32) rounded to nearest even, s = sum q_i.
 * Writes q [M][Kp], d [M][Kp/32], s [M][Kp/32]; blocks past K are zero. */
qgemv_status qgemv_quantize_act(const float* x, int64_t M, int64_t K, int64_t ldx,
                                int8_t* q, uint16_t* d, int32_t* s,
                                qgemv_stream_t stream);

/* y[n] = sum over the row's blocks of the block's integer dot with the
 * activation codes times its scales (see the format table above):
 *   Q4_0, Q8_0: y = sum_b f(dw_b) f(dx_b) D_b
 *   Q4_K: y = sum_{S,j} f(d_S) sc_Sj f(dx_b) D_Sj - f(dmin_S) m_Sj f(dx_b) s_b
 *   Q6_K: y = sum_{S,g} f(d_S) sc_Sg f(dx_b) D16_Sg   (groups of 16)
 * with D the int32 block dot of the codes (minus the format's offset) and the
 * activation codes.  w: N weight rows in the format; q/d/s: one activation
 * row from qgemv_quantize_act with the same K; y: fp32 [N].
 * The weight rows are read once, as packed bytes. */
qgemv_status qgemv_q4_0(const void* w, int64_t N, int64_t K, const int8_t* q,
                        const uint16_t* d, const int32_t* s, float* y,
                        qgemv_stream_t stream);
qgemv_status qgemv_q4_k(const void* w, int64_t N, int64_t K, const int8_t* q,
                        const uint16_t* d, const int32_t* s, float* y,
                        qgemv_stream_t stream);
qgemv_status qgemv_q6_k(const void* w, int64_t N, int64_t K, const int8_t* q,
                        const uint16_t* d, const int32_t* s, float* y,
                        qgemv_stream_t stream);
qgemv_status qgemv_q8_0(const void* w, int64_t N, int64_t K, const int8_t* q,
                        const uint16_t* d, const int32_t* s, float* y,
                        qgemv_stream_t stream);

/* A few activation rows at once against Q4_K weights (the batched prefill
 * chunk; "Backends and hardware", section "CUDA": tensor-core prefill that
 * stages the next weight tile behind the current multiply).  Row m of y
 * equals qgemv_q4_k on activation row m (colibri GPU backends, eligibility
 * gates: C = A x B is row-independent).  q [M][Kp], d/s [M][Kp/32],
 * y fp32 [M][N] row-major, 1 <= M <= QGEMV_M_MAX.
 * variant: QGEMV_VARIANT_DOT4 (4 x int8 dots: M = 1 is qgemv_q4_k itself;
 * more rows stream the weights once per group of up to four activation
 * rows, each output row then having the bits of qgemv_q4_k on its row where
 * that GEMV streams its rows, K > 2048), QGEMV_VARIANT_MFMA (int8 matrix
 * cores), or QGEMV_VARIANT_AUTO (MFMA from M = 3 where N >= 8192, i.e. at
 * least 512 tiles of 16 rows, and from M = 5 below that; DOT4 under it). */
qgemv_status qgemm_q4_k_small_m(const void* w, int64_t N, int64_t K, int64_t M,
                                const int8_t* q, const uint16_t* d, const int32_t* s,
                                float* y, int variant, qgemv_stream_t stream);

/* The same product for Q6_K and Q4_0 weights (the prefill chunk through the
 * down projection and lm_head, which are Q6_K in a Q4_K_M model; "llambda.lisp"
 * README, Features & Architecture).  Arguments, layouts, limits and errors as
 * for qgemm_q4_k_small_m; K % 32 == 0 for Q4_0, any K <= QGEMV_K_MAX.
 * variant: QGEMV_VARIANT_MFMA (int8 matrix cores), QGEMV_VARIANT_DOT4 (as
 * for Q4_K: the batch-1 GEMV at M = 1, else up to four activation rows per
 * pass of its streaming kernel, with its bits where it streams the rows; rows
 * of more than 16384 weights: the batch-1 GEMV on each row), or
 * QGEMV_VARIANT_AUTO (DOT4 up to M = 4, MFMA from M = 5). */
/* Validation: the small-M product of variant (QGEMV_VARIANT_MFMA,
 * _MFMA_STAGED or _MFMA_RESIDENT) run by the kernel that variant selects for
 * this format and shape, which also stores every raw int32 matrix-core tile
 * to dots: int32 [M][N][nb], the dots of the unsigned codes before any
 * scale, offset or min -- Q4_K: sum code*q per 32-block (nb = Kp/32);
 * Q4_0: sum code*q with codes 0..15 per 32-block, i.e. the block dot of
 * qgemv_block_dots plus 8 * s (nb = K/32); Q6_K: sum code*q with codes 0..63
 * per 16-group, i.e. qgemv_block_dots' value plus 32 * (the group's code sum)
 * (nb = Kp/16) ("Backends and hardware", section "CPU": the way to tell a
 * SIMD bug from a block bug).  y [M][N] receives the product as from the
 * small-M entry.  fmt: QGEMV_FMT_Q4_K, _Q6_K or _Q4_0.  Other variants, and
 * shapes for which the variant selects the wave-stream kernel (Q6_K from
 * M = 17 under MFMA), return QGEMV_E_UNSUPPORTED.  Other arguments, limits and
 * errors as for qgemm_q4_k_small_m. */
qgemv_status qgemm_small_m_block_dots(int fmt, const void* w, int64_t N, int64_t K,
                                     int64_t M, const int8_t* q, const uint16_t* d,
                                     const int32_t* s, float* y, int variant,
                                     int32_t* dots, qgemv_stream_t stream);

qgemv_status qgemm_q6_k_small_m(const void* w, int64_t N, int64_t K, int64_t M,
                                const int8_t* q, const uint16_t* d, const int32_t* s,
                                float* y, int variant, qgemv_stream_t stream);
qgemv_status qgemm_q4_0_small_m(const void* w, int64_t N, int64_t K, int64_t M,
                                const int8_t* q, const uint16_t* d, const int32_t* s,
                                float* y, int variant, qgemv_stream_t stream);

/* SwiGLU glue between the gate|up and down products (llambda.lisp README,
 * supported architectures; "Running an LLM on VKNN", SwiGLU):
 * gu fp32 [2N] = [gate (N) | up (N)], N % 32 == 0.
 *   h_i = g_i / (1 + exp(-g_i)) * u_i   (fp32)
 * then h is quantised exactly as qgemv_quantize_act with K = N: writes
 * q [Kp], d [Kp/32], s [Kp/32]; if h != NULL the fp32 h [N] is written too. */
qgemv_status qgemv_silu_mul_quantize(const float* gu, int64_t N, int8_t* q,
                                     uint16_t* d, int32_t* s, float* h,
                                     qgemv_stream_t stream);

/* The gate|up product, SwiGLU and the quantisation of its result in one
 * launch ("Running an LLM on VKNN", Performance: the decode step is almost
 * all matmul, and the few other ops each cost a launch; SwiGLU as in the
 * same page's model description).  Equal, bit for bit, to qgemv_q4_k on
 * the 2N rows followed by qgemv_silu_mul_quantize on its output.
 * w: Q4_K weights of 2N rows x K (gate rows 0..N-1, then up rows N..2N-1),
 *    row stride Kp/256*144 bytes, 16-byte aligned.
 * q, d, s: the activation of the gate|up product (qgemv_quantize_act, K).
 * q_out [Np], d_out [Np/32], s_out [Np/32], Np = N rounded up to 256: the
 *    activation of the next product (K = N), blocks past N written as zero;
 *    same alignment rules as q, d, s.
 * gu: NULL, or fp32 [2N] receiving [gate | up]; h: NULL, or fp32 [N].
 * N % 32 == 0, K as for qgemv_q4_k.  The caller owns every buffer; nothing
 * is allocated; gates and errors as for qgemv_q4_k. */
qgemv_status qgemv_q4_k_swiglu_quantize(const void* w, int64_t N, int64_t K,
                                        const int8_t* q, const uint16_t* d,
                                        const int32_t* s, int8_t* q_out,
                                        uint16_t* d_out, int32_t* s_out, float* gu,
                                        float* h, qgemv_stream_t stream);

/* The gate|up product above with its own activation quantisation in the same
 * launch: equal, bit for bit, to qgemv_quantize_act(x, M = 1, K) into q, d,
 * s followed by qgemv_q4_k_swiglu_quantize on those codes ("Running an LLM
 * on VKNN", Performance: every launch besides the matmuls is overhead; the
 * quantisation is the once-per-matmul step of "Backends and hardware",
 * section "CPU").  x: fp32 [K], 16-byte aligned.  q [Kp], d [Kp/32],
 * s [Kp/32] receive the codes of x (written by the kernel; nothing in the
 * launch reads them back).  Every workgroup quantises x into its own LDS
 * while its first weight rows load.  Other arguments, limits and errors as
 * for qgemv_q4_k_swiglu_quantize; x must not overlap any output. */
qgemv_status qgemv_quantize_q4_k_swiglu(const void* w, int64_t N, int64_t K,
                                        const float* x, int8_t* q, uint16_t* d,
                                        int32_t* s, int8_t* q_out, uint16_t* d_out,
                                        int32_t* s_out, float* gu, float* h,
                                        qgemv_stream_t stream);

/* Load-time repack of Q6_K weights for this device ("Backends and hardware",
 * section "Repacking is a per-device decision now": a layout is chosen per
 * device at load, the on-disk format stays the default).  Q6_K super-blocks
 * are 210 bytes, so their fields sit at 2-byte alignment; the repacked row is
 * tiles of 8 super-blocks, 1680 bytes each:
 *   ql[8][128] | qh[8][64] | sc[8][16] | d[8] (fp16 bits)
 * (super-block i of the tile keeps its ql, qh, sc and d bytes unchanged), so
 * every field starts on a 16-byte boundary (sc: 8).  A row of S = Kp/256
 * super-blocks takes ceil(S/8) * 1680 bytes -- the same as the native 210 * S
 * when S % 8 == 0 -- and the super-blocks of a partial last tile are zero.
 * w: native Q6_K [N rows], w_r: [N][ceil(S/8) * 1680] bytes; both 16-byte
 * aligned, caller-owned, not overlapping.  Gates as for qgemv_q6_k. */
qgemv_status qgemv_q6_k_repack(const void* w, int64_t N, int64_t K, void* w_r,
                               qgemv_stream_t stream);
/* qgemv_q6_k on weights repacked by qgemv_q6_k_repack (same K): the same
 * arithmetic, with every weight field read from an aligned address. */
qgemv_status qgemv_q6_k_r8(const void* w_r, int64_t N, int64_t K, const int8_t* q,
                           const uint16_t* d, const int32_t* s, float* y,
                           qgemv_stream_t stream);

/* Activation quantisation and one GEMV in a single launch: equal, bit for
 * bit, to qgemv_quantize_act(x, M = 1, K) into q, d, s followed by the GEMV
 * of format fmt (QGEMV_FMT_Q4_0, _Q4_K, _Q6_K, _Q8_0 or _Q6_K_R8 for weights
 * from qgemv_q6_k_repack) on those codes ("Running an LLM on VKNN",
 * Performance: every launch besides the matmuls is overhead; "Backends and
 * hardware", section "CPU": the activation is quantised once per matmul).
 * x: fp32 [K], 16-byte aligned; q [Kp], d [Kp/32], s [Kp/32] receive the
 * codes of x; y: fp32 [N].  One launch, in which every workgroup quantises
 * x into its own LDS while its first weight rows load -- except where the
 * staged rows and the quantised x would not fit a workgroup's LDS (the
 * longest rows, e.g. K = 32768 for Q4_K and Q6_K), which take the two
 * launches.  Other arguments, limits and errors as for the format's GEMV; x
 * must not overlap any output. */
qgemv_status qgemv_quantize_gemv(int fmt, const void* w, int64_t N, int64_t K,
                                 const float* x, int8_t* q, uint16_t* d, int32_t* s,
                                 float* y, qgemv_stream_t stream);

/* Several GEMVs on one activation row in one launch (the q/k/v projections,
 * or gate and up stored apart: "Running an LLM on VKNN", Performance: every
 * launch besides the matmuls is overhead; llambda.lisp README, Features:
 * row-parallel GEMV with isolated writes).  count matrices of one format
 * fmt and one K: w[i] (device, 16-byte aligned) holds n[i] rows, y[i]
 * (device, fp32 [n[i]]) receives their products with the activation q, d, s
 * (qgemv_quantize_act, same K).  y[i] equals the format's GEMV of matrix i
 * bit for bit.  w, n, y are host arrays of count entries, read during the
 * call only.  0 <= count <= QGEMV_MULTI_MAX (larger: QGEMV_E_UNSUPPORTED);
 * count == 0 or all n[i] == 0 is a no-op; n[i] < 0: QGEMV_E_SHAPE.  Rows of
 * at most 32 units of 64 weights (K <= 2048) go out as one launch over the
 * combined rows; longer rows take one launch per matrix.  Other gates and
 * errors as for the format's GEMV. */
qgemv_status qgemv_multi(int fmt, int count, const void* const* w, const int64_t* n,
                         int64_t K, const int8_t* q, const uint16_t* d, const int32_t* s,
                         float* const* y, qgemv_stream_t stream);
/* qgemv_multi with the activation quantised from fp32 x [K] (16-byte
 * aligned) in the same launch: equal, bit for bit, to qgemv_quantize_act
 * into q, d, s followed by qgemv_multi; q, d, s receive the codes. */
qgemv_status qgemv_quantize_multi(int fmt, int count, const void* const* w,
                                  const int64_t* n, int64_t K, const float* x, int8_t* q,
                                  uint16_t* d, int32_t* s, float* const* y,
                                  qgemv_stream_t stream);

/* Validation: the int32 block dots of weight rows [row0, row0+nrows) against
 * one activation row q [Kp], computed by the same device code as the GEMV
 * kernels.  dots: int32 [nrows][nblk] with nblk = K/32 (Q4_0, Q8_0),
 * Kp/32 (Q4_K: sub-blocks of 32, codes 0..15, no min), Kp/16 (Q6_K and
 * Q6_K_R8: groups of 16, codes minus 32); Q4_0 dots include the -8 offset.  "The way to tell a
 * SIMD bug from a block bug" ("Backends and hardware", section "CPU"). */
qgemv_status qgemv_block_dots(int fmt, const void* w, int64_t N, int64_t K,
                              int64_t row0, int64_t nrows, const int8_t* q,
                              int32_t* dots, qgemv_stream_t stream);
/* Validation: the same block dots through the loaders the streaming GEMV
 * kernels run (the same passage): each (row, split-K slice) is split into
 * wk slices as those kernels split it, staged in 16-byte chunks, parked in
 * LDS and read back field by field (including 2-byte-misaligned Q6_K, Q4_0
 * and Q8_0 fields and an empty last slice), with the activation in the same
 * registers; the dots are stored instead of scaled.  d, s: the activation's
 * fp16 scale bits and code sums (qgemv_quantize_act), which those registers
 * also hold.  wk: 1, 2 or 4; a (K, wk) whose slices exceed 128 units of 64
 * weights returns QGEMV_E_UNSUPPORTED.  Entries of dots for blocks past K are
 * not written.  Other arguments, layout, gates and errors as for
 * qgemv_block_dots. */
qgemv_status qgemv_block_dots_staged(int fmt, const void* w, int64_t N, int64_t K,
                                     int64_t row0, int64_t nrows, const int8_t* q,
                                     const uint16_t* d, const int32_t* s, int wk,
                                     int32_t* dots, qgemv_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
