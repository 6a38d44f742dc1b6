// k_gemv.hip -- batch-1 W4A8 GEMV kernels (Q4_0, Q4_K, Q6_K, Q8_0) and the
// block-dots validation kernel.
//
// Decode-time GEMV is bound by the stream of packed weight bytes from HBM
// ("Running an LLM on VKNN", Performance: the decode step is
// weight-memory-bandwidth-bound), so the kernels are shaped around reading
// every weight byte exactly once with wide loads while keeping enough bytes
// in flight:
//   * a row is split into 64-weight units (see qgemv_device.h); LPR lanes of a
//     wavefront share one row (LPR = 64 for K >= 4096, fewer for short rows,
//     so a wave then covers 64/LPR rows at once), lane i taking units
//     i, i + LPR, ...  Consecutive lanes read consecutive units, so a wave's
//     loads cover one contiguous stretch of the row.
//   * the activation row (codes, fp32 scales and per-format helpers) is staged
//     once per workgroup in LDS and shared by all rows the workgroup handles.
//   * block dots are exact int32 (v_dot4_i32_i8); scales and mins are applied
//     in fp32 per block; the LPR partial sums of a row are reduced across lanes
//     in a fixed order (deterministic), and one lane writes y[row]
//     ("llambda.lisp" README, Features: row-parallel GEMV with isolated,
//     lock-free writes).
//   * a workgroup (4 waves) owns a contiguous run of rows, so the cache lines
//     shared by neighbouring rows are fetched by one XCD.
#include "qgemv_device.h"
#include "qgemv_launch.h"

namespace qgemv {

constexpr int WG = 256;  // 4 wavefronts of 64

// LDS layout of the staged activation row (Kp codes, then per-block data).
struct ActSmem {
    const uint8_t* codes;  // [Kp]
    const float* dx;       // [Kp/32] fp32 value of the block scale
    const float* dxs;      // Q4_K: [Kp/32] dx * s (exact in fp32)
    const int* init;       // Q4_0: [Kp/32] -8*s ; Q6_K: [Kp/16] -32*sum16
};

__host__ __device__ inline int smem_bytes(int fmt, int Kp) {
    const int nb = Kp / 32;
    int bytes = Kp + 4 * nb;
    if (fmt == QGEMV_FMT_Q4_K || fmt == QGEMV_FMT_Q4_0) bytes += 4 * nb;
    if (fmt == QGEMV_FMT_Q6_K) bytes += 8 * nb;
    return bytes;
}

template <int FMT>
__device__ __forceinline__ ActSmem stage_act(uint8_t* smem, const int8_t* __restrict__ q,
                                             const uint16_t* __restrict__ d,
                                             const int32_t* __restrict__ s, int Kp) {
    const int nb = Kp / 32;
    uint8_t* codes = smem;
    float* dx = reinterpret_cast<float*>(smem + Kp);
    float* aux_f = dx + nb;
    int* aux_i = reinterpret_cast<int*>(dx + nb);
    const int tid = threadIdx.x;
    for (int i = tid; i < Kp / 16; i += WG)
        reinterpret_cast<u32x4*>(codes)[i] = reinterpret_cast<const u32x4*>(q)[i];
    for (int b = tid; b < nb; b += WG) {
        const float f = h2f(d[b]);
        dx[b] = f;
        if (FMT == QGEMV_FMT_Q4_K) aux_f[b] = f * (float)s[b];
        if (FMT == QGEMV_FMT_Q4_0) aux_i[b] = -8 * s[b];
    }
    if (FMT == QGEMV_FMT_Q6_K) {
        for (int g = tid; g < 2 * nb; g += WG) {
            const u32x4 v = reinterpret_cast<const u32x4*>(q)[g];
            aux_i[g] = -32 * sum16(v.x, v.y, v.z, v.w);
        }
    }
    __syncthreads();
    return ActSmem{codes, dx, aux_f, aux_i};
}

__device__ __forceinline__ void lds_act64(const uint8_t* codes, int off, Act16& x) {
    const u32x4* p = reinterpret_cast<const u32x4*>(codes + off);
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const u32x4 v = p[k];
        x.a[4 * k + 0] = v.x;
        x.a[4 * k + 1] = v.y;
        x.a[4 * k + 2] = v.z;
        x.a[4 * k + 3] = v.w;
    }
}

__device__ __forceinline__ void lds_act_q6k(const uint8_t* codes, int u, Act16& x) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(codes + Q6K::act_offset(u, j));
        x.a[4 * j + 0] = v.x;
        x.a[4 * j + 1] = v.y;
        x.a[4 * j + 2] = v.z;
        x.a[4 * j + 3] = v.w;
    }
}

// fp32 contribution of one unit of a row.
template <int FMT>
__device__ __forceinline__ float unit_term(const uint8_t* __restrict__ rp, int u, int nbw,
                                           const ActSmem& A) {
    Act16 x;
    if constexpr (FMT == QGEMV_FMT_Q4_K) {
        Q4K::W w;
        Q4K::load(rp, u, w);
        lds_act64(A.codes, 64 * u, x);
        int D[2];
        Q4K::dots(w, x, D);
        const float fd = h2f(w.hdr.x & 0xFFFFu), fdm = h2f(w.hdr.x >> 16);
        const int c = u & 3;
        float t = 0.0f;
#pragma unroll
        for (int jj = 0; jj < 2; jj++) {
            int sc, mn;
            Q4K::scale_min(w, 2 * c + jj, sc, mn);
            const int b = 2 * u + jj;
            t = fmaf((float)D[jj], fd * (float)sc * A.dx[b], t);
            t = fmaf(-(fdm * (float)mn), A.dxs[b], t);
        }
        return t;
    } else if constexpr (FMT == QGEMV_FMT_Q6_K) {
        Q6K::W w;
        Q6K::load(rp, u, w);
        lds_act_q6k(A.codes, u, x);
        int init[4], D[4];
#pragma unroll
        for (int j = 0; j < 4; j++) init[j] = A.init[Q6K::act_offset(u, j) >> 4];
        Q6K::dots(w, x, init, D);
        const float fd = h2f(w.d);
        float t = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int b = Q6K::act_offset(u, j) >> 5;
            t = fmaf((float)D[j], fd * (float)Q6K::scale(w, u, j) * A.dx[b], t);
        }
        return t;
    } else if constexpr (FMT == QGEMV_FMT_Q4_0) {
        const bool has1 = 2 * u + 1 < nbw;
        Q40::W w;
        Q40::load(rp, u, has1, w);
        lds_act64(A.codes, 64 * u, x);
        int init[2] = {A.init[2 * u], A.init[2 * u + 1]}, D[2];
        Q40::dots(w, x, init, D);
        float t = (float)D[0] * (h2f(w.d0) * A.dx[2 * u]);
        if (has1) t = fmaf((float)D[1], h2f(w.d1) * A.dx[2 * u + 1], t);
        return t;
    } else {
        const bool has1 = 2 * u + 1 < nbw;
        Q80::W w;
        Q80::load(rp, u, has1, w);
        lds_act64(A.codes, 64 * u, x);
        int D[2];
        Q80::dots(w, x, D);
        float t = (float)D[0] * (h2f(w.d0) * A.dx[2 * u]);
        if (has1) t = fmaf((float)D[1], h2f(w.d1) * A.dx[2 * u + 1], t);
        return t;
    }
}

// One workgroup = 4 waves; wave-iteration it handles rows
// base + it*4*RPW + wave*RPW + lane/LPR, for it < R.
template <int FMT, int LPR>
__global__ __launch_bounds__(WG) void k_gemv(const uint8_t* __restrict__ w, int N, int Kp,
                                              int U, int nbw, int row_bytes,
                                              const int8_t* __restrict__ q,
                                              const uint16_t* __restrict__ d,
                                              const int32_t* __restrict__ s,
                                              float* __restrict__ y, int R) {
    extern __shared__ __align__(16) uint8_t smem[];
    const ActSmem A = stage_act<FMT>(smem, q, d, s, Kp);
    constexpr int RPW = 64 / LPR;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane % LPR;
    const int64_t base = (int64_t)blockIdx.x * R * 4 * RPW + wave * RPW + lane / LPR;
    for (int it = 0; it < R; it++) {
        const int64_t row = base + (int64_t)it * 4 * RPW;
        float acc = 0.0f;
        if (row < N) {
            const uint8_t* rp = w + row * (int64_t)row_bytes;
            for (int u = li; u < U; u += LPR) acc += unit_term<FMT>(rp, u, nbw, A);
        }
#pragma unroll
        for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
        if (li == 0 && row < N) y[row] = acc;
    }
}

// Block-dots validation kernel: one thread per (row, unit); the activation is
// read from global memory, the weights with the same unit loaders and the
// integer dots with the same unit dot functions as the GEMV kernels.
template <int FMT>
__global__ __launch_bounds__(WG) void k_block_dots(const uint8_t* __restrict__ w, int64_t row0,
                                                    int64_t nrows, int U, int nbw,
                                                    int row_bytes, int nblk,
                                                    const int8_t* __restrict__ q,
                                                    int32_t* __restrict__ dots) {
    const int64_t t = (int64_t)blockIdx.x * WG + threadIdx.x;
    if (t >= nrows * U) return;
    const int64_t rr = t / U;
    const int u = (int)(t % U);
    const uint8_t* rp = w + (row0 + rr) * (int64_t)row_bytes;
    int32_t* out = dots + rr * nblk;
    Act16 x;
    if constexpr (FMT == QGEMV_FMT_Q6_K) {
        int init[4], D[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(q + Q6K::act_offset(u, j));
            x.a[4 * j] = v.x;
            x.a[4 * j + 1] = v.y;
            x.a[4 * j + 2] = v.z;
            x.a[4 * j + 3] = v.w;
            init[j] = -32 * sum16(v.x, v.y, v.z, v.w);
        }
        Q6K::W wv;
        Q6K::load(rp, u, wv);
        Q6K::dots(wv, x, init, D);
#pragma unroll
        for (int j = 0; j < 4; j++) out[Q6K::act_offset(u, j) >> 4] = D[j];
    } else {
        const u32x4* p = reinterpret_cast<const u32x4*>(q + 64 * u);
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const u32x4 v = p[k];
            x.a[4 * k] = v.x;
            x.a[4 * k + 1] = v.y;
            x.a[4 * k + 2] = v.z;
            x.a[4 * k + 3] = v.w;
        }
        int D[2];
        bool has1 = true;
        if constexpr (FMT == QGEMV_FMT_Q4_K) {
            Q4K::W wv;
            Q4K::load(rp, u, wv);
            Q4K::dots(wv, x, D);
        } else if constexpr (FMT == QGEMV_FMT_Q4_0) {
            has1 = 2 * u + 1 < nbw;
            // -8 * (sum of the block's codes): the offset of the stored code
            const int init[2] = {-8 * sum16(x.a[0], x.a[1], x.a[2], x.a[3]) -
                                     8 * sum16(x.a[4], x.a[5], x.a[6], x.a[7]),
                                 -8 * sum16(x.a[8], x.a[9], x.a[10], x.a[11]) -
                                     8 * sum16(x.a[12], x.a[13], x.a[14], x.a[15])};
            Q40::W wv;
            Q40::load(rp, u, has1, wv);
            Q40::dots(wv, x, init, D);
        } else {
            has1 = 2 * u + 1 < nbw;
            Q80::W wv;
            Q80::load(rp, u, has1, wv);
            Q80::dots(wv, x, D);
        }
        out[2 * u] = D[0];
        if (has1) out[2 * u + 1] = D[1];
    }
}

// ------------------------------------------------------------- launchers --

static int row_bytes_of(int fmt, int64_t K) {
    const int64_t Kp = (K + 255) / 256 * 256;
    switch (fmt) {
    case QGEMV_FMT_Q4_0: return (int)(K / 32 * 18);
    case QGEMV_FMT_Q8_0: return (int)(K / 32 * 34);
    case QGEMV_FMT_Q4_K: return (int)(Kp / 256 * 144);
    default: return (int)(Kp / 256 * 210);
    }
}

static int units_of(int fmt, int64_t K) {
    const int64_t Kp = (K + 255) / 256 * 256;
    if (fmt == QGEMV_FMT_Q4_K || fmt == QGEMV_FMT_Q6_K) return (int)(Kp / 64);
    return (int)((K + 63) / 64);
}

template <int FMT, int LPR>
static hipError_t launch_gemv_lpr(const GemvArgs& a, int U, int Kp, hipStream_t st) {
    constexpr int RPW = 64 / LPR;
    const int64_t rows_per_pass = 4LL * RPW;
    // Rows per wave: enough workgroups to fill the chip several times over
    // (about 2048), more rows per wave only when N is large.
    int64_t passes = (a.N + rows_per_pass - 1) / rows_per_pass;
    int R = (int)(passes / 2048);
    if (R < 1) R = 1;
    if (R > 16) R = 16;
    const int64_t grid = (passes + R - 1) / R;
    const int smem = smem_bytes(FMT, Kp);
    hipLaunchKernelGGL((k_gemv<FMT, LPR>), dim3((unsigned)grid), dim3(WG), smem, st,
                       (const uint8_t*)a.w, (int)a.N, Kp, U, (int)(a.K / 32),
                       row_bytes_of(FMT, a.K), a.q, a.d, a.s, a.y, R);
    return hipGetLastError();
}

template <int FMT>
static hipError_t launch_gemv_fmt(const GemvArgs& a, hipStream_t st) {
    const int U = units_of(FMT, a.K);
    const int Kp = (int)((a.K + 255) / 256 * 256);
    if (U > 32) return launch_gemv_lpr<FMT, 64>(a, U, Kp, st);
    if (U > 16) return launch_gemv_lpr<FMT, 32>(a, U, Kp, st);
    if (U > 8) return launch_gemv_lpr<FMT, 16>(a, U, Kp, st);
    if (U > 4) return launch_gemv_lpr<FMT, 8>(a, U, Kp, st);
    return launch_gemv_lpr<FMT, 4>(a, U, Kp, st);
}

int gemv_smem_bytes(int fmt, int64_t K) {
    return smem_bytes(fmt, (int)((K + 255) / 256 * 256));
}

hipError_t launch_gemv(int fmt, const GemvArgs& a, hipStream_t st) {
    switch (fmt) {
    case QGEMV_FMT_Q4_0: return launch_gemv_fmt<QGEMV_FMT_Q4_0>(a, st);
    case QGEMV_FMT_Q4_K: return launch_gemv_fmt<QGEMV_FMT_Q4_K>(a, st);
    case QGEMV_FMT_Q6_K: return launch_gemv_fmt<QGEMV_FMT_Q6_K>(a, st);
    default: return launch_gemv_fmt<QGEMV_FMT_Q8_0>(a, st);
    }
}

hipError_t launch_block_dots(int fmt, const void* w, int64_t K, int64_t row0, int64_t nrows,
                             const int8_t* q, int32_t* dots, hipStream_t st) {
    const int U = units_of(fmt, K);
    const int nbw = (int)(K / 32);
    const int rb = row_bytes_of(fmt, K);
    const int64_t Kp = (K + 255) / 256 * 256;
    int nblk = (fmt == QGEMV_FMT_Q6_K) ? (int)(Kp / 16)
                                        : (fmt == QGEMV_FMT_Q4_K ? (int)(Kp / 32) : nbw);
    const int64_t grid = (nrows * U + WG - 1) / WG;
    const uint8_t* wp = (const uint8_t*)w;
    switch (fmt) {
    case QGEMV_FMT_Q4_0:
        hipLaunchKernelGGL(k_block_dots<QGEMV_FMT_Q4_0>, dim3((unsigned)grid), dim3(WG), 0, st,
                           wp, row0, nrows, U, nbw, rb, nblk, q, dots);
        break;
    case QGEMV_FMT_Q4_K:
        hipLaunchKernelGGL(k_block_dots<QGEMV_FMT_Q4_K>, dim3((unsigned)grid), dim3(WG), 0, st,
                           wp, row0, nrows, U, nbw, rb, nblk, q, dots);
        break;
    case QGEMV_FMT_Q6_K:
        hipLaunchKernelGGL(k_block_dots<QGEMV_FMT_Q6_K>, dim3((unsigned)grid), dim3(WG), 0, st,
                           wp, row0, nrows, U, nbw, rb, nblk, q, dots);
        break;
    default:
        hipLaunchKernelGGL(k_block_dots<QGEMV_FMT_Q8_0>, dim3((unsigned)grid), dim3(WG), 0, st,
                           wp, row0, nrows, U, nbw, rb, nblk, q, dots);
        break;
    }
    return hipGetLastError();
}

}  // namespace qgemv
