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

// The integer block dots of one unit from its loaded fields and its
// activation registers: the dot functions that Unit<FMT>::term calls, with
// the ints kept.  NB blocks per unit; blk(u, j) is the output column of
// block j of unit u.
template <int FMT>
struct UnitDots;
template <>
struct UnitDots<QGEMV_FMT_Q4_K> {
    static constexpr int NB = 2;
    __device__ static void dots(const Q4K::W& w, const ActReg<QGEMV_FMT_Q4_K>& a, int D[4]) {
        Q4K::dots(w, a.x, D);
    }
    __device__ static int blk(int u, int j) { return 2 * u + j; }
};
template <>
struct UnitDots<QGEMV_FMT_Q6_K> {
    static constexpr int NB = 4;
    __device__ static void dots(const Q6K::W& w, const ActReg<QGEMV_FMT_Q6_K>& a, int D[4]) {
        Q6K::dots(w, a.x, a.init, D);
    }
    __device__ static int blk(int u, int j) { return Q6K::act_offset(u, j) >> 4; }
};
template <>
struct UnitDots<QGEMV_FMT_Q6_K_R8> : UnitDots<QGEMV_FMT_Q6_K> {};
template <>
struct UnitDots<QGEMV_FMT_Q4_0> {
    static constexpr int NB = 2;
    __device__ static void dots(const Q40::W& w, const ActReg<QGEMV_FMT_Q4_0>& a, int D[4]) {
        Q40::dots(w, a.x, a.init, D);
    }
    __device__ static int blk(int u, int j) { return 2 * u + j; }
};
template <>
struct UnitDots<QGEMV_FMT_Q8_0> {
    static constexpr int NB = 2;
    __device__ static void dots(const Q80::W& w, const ActReg<QGEMV_FMT_Q8_0>& a, int D[4]) {
        Q80::dots(w, a.x, D);
    }
    __device__ static int blk(int u, int j) { return 2 * u + j; }
};

// Block-dots validation through the LDS-streaming path: one wave per (row,
// split-K slice), the slice split, staged, parked in LDS and read back by the
// same SliceStream and UnitLds code as k_gemv_lds and k_gemv_dyn (16-byte
// chunk grid, shifted last chunk, misaligned-field readers, empty last
// slice), the activation in the same registers; only the last step differs:
// the unit's integer dots are stored instead of scaled.  Lanes past the
// slice and blocks past K store nothing.
template <int FMT, int UPL, int NL>
__global__ __launch_bounds__(WG) void k_block_dots_staged(const uint8_t* __restrict__ w,
                                                           int64_t row0, int64_t nrows, int U,
                                                           int US, int WK, int nbw,
                                                           int row_bytes, int buf_bytes, int nblk,
                                                           const int8_t* __restrict__ q,
                                                           const uint16_t* __restrict__ d,
                                                           const int32_t* __restrict__ s,
                                                           int32_t* __restrict__ dots) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t t = (int64_t)blockIdx.x * (WG / 64) + wave;
    if (t >= nrows * WK) return;   // whole waves; no workgroup barrier follows
    const int64_t rr = t / WK;
    const int kq = (int)(t % WK);
    SliceStream<FMT, UPL, NL, kStreamNT> ss(lane, U, US, kq, nbw, row_bytes);
    ss.load_act(q, d, s);
    u32x4 R[NL];
    const int delta = ss.stage(R, w + (row0 + rr) * (int64_t)row_bytes);
    uint8_t* buf = lds + wave * buf_bytes;
    ss.commit(R, delta, buf);
    int32_t* out = dots + rr * nblk;
#pragma unroll
    for (int i = 0; i < UPL; i++) {
        typename Unit<FMT>::W wv;
        UnitLds<FMT>::load(buf, delta, ss.ul[i], ss.has1[i], wv);
        int D[4];
        UnitDots<FMT>::dots(wv, ss.A[0][i], D);
        const int u = ss.u_lo + ss.ul[i];
        constexpr bool PAIR = FMT == QGEMV_FMT_Q4_0 || FMT == QGEMV_FMT_Q8_0;
        if (ss.ok[i]) {
#pragma unroll
            for (int j = 0; j < UnitDots<FMT>::NB; j++)
                if (!PAIR || j == 0 || ss.has1[i]) out[UnitDots<FMT>::blk(u, j)] = D[j];
        }
    }
}

template <int FMT>
static int staged_nl(int64_t K, int WK, int& US, int& buf_bytes, int& upl) {
    const int U = units_of(FMT, K);
    const SliceGeom g = slice_geom<FMT>(K, U, WK);
    US = g.US;
    buf_bytes = 16 * g.nchunk + 16;
    upl = (US + 63) / 64;
    return (g.nchunk + 63) / 64;
}

template <int FMT>
static bool staged_ok(int64_t K, int WK) {
    int US, bb, upl;
    const int nl = staged_nl<FMT>(K, WK, US, bb, upl);
    return upl <= 2 && nl <= 8;
}

bool block_dots_staged_supported(int fmt, int64_t K, int wk) {
    if (wk != 1 && wk != 2 && wk != 4) return false;
    switch (fmt) {
    case QGEMV_FMT_Q4_0: return staged_ok<QGEMV_FMT_Q4_0>(K, wk);
    case QGEMV_FMT_Q4_K: return staged_ok<QGEMV_FMT_Q4_K>(K, wk);
    case QGEMV_FMT_Q6_K: return staged_ok<QGEMV_FMT_Q6_K>(K, wk);
    case QGEMV_FMT_Q6_K_R8: return staged_ok<QGEMV_FMT_Q6_K_R8>(K, wk);
    default: return staged_ok<QGEMV_FMT_Q8_0>(K, wk);
    }
}

template <int FMT, int UPL, int NL>
static void launch_staged_cfg(const uint8_t* w, int64_t K, int64_t row0, int64_t nrows, int WK,
                              int US, int buf_bytes, int nblk, const int8_t* q,
                              const uint16_t* d, const int32_t* s, int32_t* dots,
                              hipStream_t st) {
    const int64_t grid = (nrows * WK + WG / 64 - 1) / (WG / 64);
    launch_kernel(k_block_dots_staged<FMT, UPL, NL>, dim3((unsigned)grid), dim3(WG),
                  (unsigned)(WG / 64 * buf_bytes), st, w, row0, nrows, units_of(FMT, K), US, WK,
                  (int)(K / 32), row_bytes_of(FMT, K), buf_bytes, nblk, q, d, s, dots);
}

template <int FMT>
static hipError_t launch_staged_fmt(const uint8_t* w, int64_t K, int64_t row0, int64_t nrows,
                                    int WK, int nblk, const int8_t* q, const uint16_t* d,
                                    const int32_t* s, int32_t* dots, hipStream_t st) {
    int US, bb, upl;
    const int nl = staged_nl<FMT>(K, WK, US, bb, upl);
    if (upl > 2 || nl > 8) return hipErrorInvalidValue;
    // more chunks per lane than a slice needs only repeat its last chunk
    if (upl == 1 && nl <= 2)
        launch_staged_cfg<FMT, 1, 2>(w, K, row0, nrows, WK, US, bb, nblk, q, d, s, dots, st);
    else if (upl == 1 && nl <= 4)
        launch_staged_cfg<FMT, 1, 4>(w, K, row0, nrows, WK, US, bb, nblk, q, d, s, dots, st);
    else if (upl == 1)
        launch_staged_cfg<FMT, 1, 8>(w, K, row0, nrows, WK, US, bb, nblk, q, d, s, dots, st);
    else if (nl <= 4)
        launch_staged_cfg<FMT, 2, 4>(w, K, row0, nrows, WK, US, bb, nblk, q, d, s, dots, st);
    else
        launch_staged_cfg<FMT, 2, 8>(w, K, row0, nrows, WK, US, bb, nblk, q, d, s, dots, st);
    return hipGetLastError();
}

hipError_t launch_block_dots_staged(int fmt, const void* w, int64_t K, int64_t row0,
                                    int64_t nrows, const int8_t* q, const uint16_t* d,
                                    const int32_t* s, int wk, int32_t* dots, hipStream_t st) {
    const int64_t Kp = (K + 255) / 256 * 256;
    const int nblk = (fmt == QGEMV_FMT_Q6_K || fmt == QGEMV_FMT_Q6_K_R8)
                         ? (int)(Kp / 16)
                         : (fmt == QGEMV_FMT_Q4_K ? (int)(Kp / 32) : (int)(K / 32));
    const uint8_t* wp = (const uint8_t*)w;
    switch (fmt) {
    case QGEMV_FMT_Q4_0:
        return launch_staged_fmt<QGEMV_FMT_Q4_0>(wp, K, row0, nrows, wk, nblk, q, d, s, dots, st);
    case QGEMV_FMT_Q4_K:
        return launch_staged_fmt<QGEMV_FMT_Q4_K>(wp, K, row0, nrows, wk, nblk, q, d, s, dots, st);
    case QGEMV_FMT_Q6_K:
        return launch_staged_fmt<QGEMV_FMT_Q6_K>(wp, K, row0, nrows, wk, nblk, q, d, s, dots, st);
    case QGEMV_FMT_Q6_K_R8:
        return launch_staged_fmt<QGEMV_FMT_Q6_K_R8>(wp, K, row0, nrows, wk, nblk, q, d, s, dots,
                                                    st);
    default:
        return launch_staged_fmt<QGEMV_FMT_Q8_0>(wp, K, row0, nrows, wk, nblk, q, d, s, dots, st);
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
