// k_gemv.hip -- dispatch of the batch-1 GEMV launchers by weight format, the
// Q6_K load-time repack, and the block-dots validation kernel.  The kernels
// and their per-format launchers are in k_gemv.h and k_gemv_<fmt>.hip.
#include "k_gemv.h"

namespace qgemv {

hipError_t launch_multi(int fmt, const MultiRows& mr, int64_t K, const int8_t* q,
                        const uint16_t* d, const int32_t* s, hipStream_t st) {
    switch (fmt) {
    case QGEMV_FMT_Q4_0: return launch_multi_q4_0(mr, K, q, d, s, st);
    case QGEMV_FMT_Q4_K: return launch_multi_q4_k(mr, K, q, d, s, st);
    case QGEMV_FMT_Q6_K: return launch_multi_q6_k(mr, K, q, d, s, st);
    case QGEMV_FMT_Q6_K_R8: return launch_multi_q6_k_r8(mr, K, q, d, s, st);
    default: return launch_multi_q8_0(mr, K, q, d, s, st);
    }
}

hipError_t launch_quantize_multi(int fmt, const MultiRows& mr, int64_t K, const ActIn& ai,
                                 hipStream_t st) {
    switch (fmt) {
    case QGEMV_FMT_Q4_0: return launch_quantize_multi_q4_0(mr, K, ai, st);
    case QGEMV_FMT_Q4_K: return launch_quantize_multi_q4_k(mr, K, ai, st);
    case QGEMV_FMT_Q6_K: return launch_quantize_multi_q6_k(mr, K, ai, st);
    case QGEMV_FMT_Q6_K_R8: return launch_quantize_multi_q6_k_r8(mr, K, ai, st);
    default: return launch_quantize_multi_q8_0(mr, K, ai, st);
    }
}

hipError_t launch_gemv(int fmt, const GemvArgs& a, hipStream_t st) {
    switch (fmt) {
    case QGEMV_FMT_Q4_0: return launch_gemv_q4_0(a, st);
    case QGEMV_FMT_Q4_K: return launch_gemv_q4_k(a, st);
    case QGEMV_FMT_Q6_K: return launch_gemv_q6_k(a, st);
    case QGEMV_FMT_Q6_K_R8: return launch_gemv_q6_k_r8(a, st);
    default: return launch_gemv_q8_0(a, st);
    }
}

hipError_t launch_quantize_gemv(int fmt, const GemvArgs& a, const ActIn& ai, hipStream_t st) {
    switch (fmt) {
    case QGEMV_FMT_Q4_0: return launch_quantize_gemv_q4_0(a, ai, st);
    case QGEMV_FMT_Q4_K: return launch_quantize_gemv_q4_k(a, ai, st);
    case QGEMV_FMT_Q6_K: return launch_quantize_gemv_q6_k(a, ai, st);
    case QGEMV_FMT_Q6_K_R8: return launch_quantize_gemv_q6_k_r8(a, ai, st);
    default: return launch_quantize_gemv_q8_0(a, ai, st);
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
    if constexpr (FMT == QGEMV_FMT_Q6_K || FMT == QGEMV_FMT_Q6_K_R8) {
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
        if (FMT == QGEMV_FMT_Q6_K_R8) Q6K::load_r8(rp, u, wv);
        else Q6K::load(rp, u, wv);
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

// Q6_K -> Q6_K_R8: one thread per (row, tile slot); a slot past the row's
// super-blocks (the rest of a partial last tile) is written as zeros.  The
// native super-block is 2-byte aligned, so it is copied as 16-bit words.
__global__ __launch_bounds__(WG) void k_q6k_repack(const uint8_t* __restrict__ w, int64_t N,
                                                   int nsb, int64_t row_bytes, int ntile,
                                                   uint8_t* __restrict__ wr) {
    const int64_t gt = (int64_t)blockIdx.x * WG + threadIdx.x;
    const int64_t slots = (int64_t)ntile * Q6K::TILE_SB;
    if (gt >= N * slots) return;
    const int64_t r = gt / slots;
    const int slot = (int)(gt - r * slots);
    const int T = slot >> 3, i = slot & 7, S = slot;
    uint8_t* tile = wr + r * (int64_t)ntile * Q6K::TILE_BYTES + (int64_t)T * Q6K::TILE_BYTES;
    uint16_t* ql = reinterpret_cast<uint16_t*>(tile + 128 * i);
    uint16_t* qh = reinterpret_cast<uint16_t*>(tile + Q6K::T_QH + 64 * i);
    uint16_t* sc = reinterpret_cast<uint16_t*>(tile + Q6K::T_SC + 16 * i);
    uint16_t* dd = reinterpret_cast<uint16_t*>(tile + Q6K::T_D + 2 * i);
    if (S < nsb) {
        const uint16_t* src = reinterpret_cast<const uint16_t*>(w + r * row_bytes + 210 * S);
        for (int k = 0; k < 64; k++) ql[k] = src[k];
        for (int k = 0; k < 32; k++) qh[k] = src[64 + k];
        for (int k = 0; k < 8; k++) sc[k] = src[96 + k];
        dd[0] = src[104];
    } else {
        for (int k = 0; k < 64; k++) ql[k] = 0;
        for (int k = 0; k < 32; k++) qh[k] = 0;
        for (int k = 0; k < 8; k++) sc[k] = 0;
        dd[0] = 0;
    }
}

hipError_t launch_q6k_repack(const void* w, int64_t N, int64_t K, void* wr, hipStream_t st) {
    const int nsb = (int)((K + 255) / 256);
    const int ntile = (nsb + Q6K::TILE_SB - 1) / Q6K::TILE_SB;
    const int64_t threads = N * ntile * Q6K::TILE_SB;
    const int64_t grid = (threads + WG - 1) / WG;
    launch_kernel(k_q6k_repack, dim3((unsigned)grid), dim3(WG), 0, st, (const uint8_t*)w, N,
                  nsb, (int64_t)nsb * 210, ntile, (uint8_t*)wr);
    return hipGetLastError();
}

hipError_t launch_block_dots(int fmt, const void* w, int64_t K, int64_t row0, int64_t nrows,
                             const int8_t* q, int32_t* dots, hipStream_t st) {
    const int U = units_of(fmt, K);
    const int nbw = (int)(K / 32);
    const int rb = row_bytes_of(fmt, K);
    const int64_t Kp = (K + 255) / 256 * 256;
    int nblk = (fmt == QGEMV_FMT_Q6_K || fmt == QGEMV_FMT_Q6_K_R8) ? (int)(Kp / 16)
                                        : (fmt == QGEMV_FMT_Q4_K ? (int)(Kp / 32) : nbw);
    const int64_t grid = (nrows * U + WG - 1) / WG;
    const uint8_t* wp = (const uint8_t*)w;
    switch (fmt) {
    case QGEMV_FMT_Q4_0:
        launch_kernel(k_block_dots<QGEMV_FMT_Q4_0>, dim3((unsigned)grid), dim3(WG), 0, st,
                      wp, row0, nrows, U, nbw, rb, nblk, q, dots);
        break;
    case QGEMV_FMT_Q4_K:
        launch_kernel(k_block_dots<QGEMV_FMT_Q4_K>, dim3((unsigned)grid), dim3(WG), 0, st,
                      wp, row0, nrows, U, nbw, rb, nblk, q, dots);
        break;
    case QGEMV_FMT_Q6_K:
        launch_kernel(k_block_dots<QGEMV_FMT_Q6_K>, dim3((unsigned)grid), dim3(WG), 0, st,
                      wp, row0, nrows, U, nbw, rb, nblk, q, dots);
        break;
    case QGEMV_FMT_Q6_K_R8:
        launch_kernel(k_block_dots<QGEMV_FMT_Q6_K_R8>, dim3((unsigned)grid), dim3(WG), 0,
                      st, wp, row0, nrows, U, nbw, rb, nblk, q, dots);
        break;
    default:
        launch_kernel(k_block_dots<QGEMV_FMT_Q8_0>, dim3((unsigned)grid), dim3(WG), 0, st,
                      wp, row0, nrows, U, nbw, rb, nblk, q, dots);
        break;
    }
    return hipGetLastError();
}

}  // namespace qgemv
