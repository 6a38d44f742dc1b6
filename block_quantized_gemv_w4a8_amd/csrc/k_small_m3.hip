// k_small_m3.hip -- the small-M product for up to 16 activation rows on the
// int8 matrix cores, with the activation resident in registers.
//
// Row m of y equals the batch-1 GEMV of activation row m (colibri GPU
// backends, eligibility gates: C = A x B is row-independent); each 32-wide K
// block gets its own exact int32 dot on v_mfma_i32_16x16x32_i8 because the
// weights and the activation both carry a scale per block, and the fp32
// epilogue applies the scales ("Backends and hardware", section "CUDA": the
// prefill kernel's gap is keeping the next weight tile streaming behind the
// current multiply).
//
// Work split.  One workgroup of 8 waves per compute unit takes the 16-row
// weight tiles b, b + G, b + 2G, ...; wave w owns the w-th of 8 slices of K
// (whole super-blocks) for every tile, so the A operands of its slice -- the
// activation codes of all (up to 16) rows -- are loaded once and stay in
// VGPRs.  The wave streams its slice of each tile with 16-byte loads (a wave
// instruction covers about 1 KB of consecutive row bytes), DEPTH stages ahead,
// parks a stage in its own LDS buffer and reads the B operands back in the
// MFMA layout; no other wave waits for it.  The activation scales (fp32 dx
// and dx * s per block and row) sit in LDS for the whole kernel.  Once per
// tile the 8 waves meet: each parks its 16 x 16 partial sums, and the sum
// over the slices is taken in slice order and stored.
//
// Per format, with D the 16 x 16 int32 tile of one 32-block:
//   Q4_K  y += d*sc_j*dx*D  - (dmin*m_j)(dx*s)
// The min term is a small dense product over the blocks of a super-block and
// goes to the fp32 MFMA (v_mfma_f32_16x16x4f32, four blocks per
// instruction).  Lane l: activation row l % 16 and weight row l % 16 for the
// operands, K quarter l / 16 of each block; its outputs are activation rows
// 4 (l / 16) + i of weight row l % 16.
#include <utility>

#include "qgemv_device.h"
#include "qgemv_launch.h"

namespace qgemv {
namespace sm3 {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NTH = 512;                 // 8 waves
constexpr int NW = NTH / 64;
constexpr int NSP = 1;                   // super-blocks per stage
constexpr int DEPTH = 4;                 // stages in flight per wave
constexpr int SBB = 144;                 // bytes of a Q4_K super-block
constexpr int SPAN = NSP * SBB;          // row bytes of a stage
constexpr int NCH = SPAN / 16;           // 16-byte chunks of a row's stage
constexpr int TCH = 16 * NCH;            // chunks of a tile's stage
constexpr int LPT = (TCH + 63) / 64;     // loads per lane and stage
constexpr int WSTR = SPAN + 16;          // LDS row stride of a wave's buffer (40 dwords)
constexpr int WBUF = 16 * WSTR;          // a wave's stage buffer
constexpr int SLOT = NW * 256 * 4;       // partial sums of one tile

// LDS-only workgroup barrier: every wave's LDS writes are visible after it
// (global memory is not involved, so outstanding loads are not waited for).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Wave-private LDS: this wave's own writes are visible to its own reads.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// f(integral_constant<int, i>) for i = 0 .. N-1, in order
template <int... I, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, I...>, F&& f) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

// NST: stages per wave slice (the slice holds at most NST * NSP
// super-blocks).  LDS: the 8 stage buffers, dx and dx*s of every block and
// row ([block][row], fp32), two tiles' partial-sum slots.
// DOTS (validation): every int32 MFMA tile is also stored to dots [M][N][Kp/32],
// the raw dots of the unsigned codes before any scale or min.
template <int NST, bool DOTS = false>
__global__ __launch_bounds__(NTH) void k_sm3_q4k(const uint8_t* __restrict__ w, int N, int Kp,
                                                 int M, const int8_t* __restrict__ q,
                                                 const uint16_t* __restrict__ d,
                                                 const int32_t* __restrict__ s,
                                                 float* __restrict__ y, int32_t* __restrict__ dots) {
    constexpr int NBMAX = NW * NST * NSP * 8;   // blocks of the longest row taken
    __shared__ __align__(16) uint8_t wbuf[NW * WBUF];
    __shared__ __align__(16) float dxl[NBMAX * 16];
    __shared__ __align__(16) float dxsl[NBMAX * 16];
    __shared__ __align__(16) float slot[2][NW * 256];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g = lane >> 4;
    const int nsb = Kp / 256, nb = Kp / 32;
    const int spw = (nsb + NW - 1) / NW;          // super-blocks per slice
    const int sb0 = wave * spw;                   // this wave's first super-block
    const int sb1 = min(sb0 + spw, nsb);          // its end (<= sb0: empty slice)
    const int64_t row_bytes = (int64_t)nsb * SBB;
    const int G = gridDim.x, b = blockIdx.x;
    const int ntiles = (N + 15) / 16;
    const int ntk = b < ntiles ? (ntiles - b + G - 1) / G : 0;   // this workgroup's tiles
    const int nit = ntk * NST;                                   // (tile, stage) items

    // activation scales of every block and row (rows past M: zero): a
    // thread takes 8 consecutive blocks of one row with 16-byte loads (rows
    // of d and s start 16-byte aligned: nb is a multiple of 8), every load
    // of a pass issued before any is used
    {
        constexpr int PASSES = (NBMAX * 2 + NTH - 1) / NTH;   // 16 rows x nb/8 groups
#pragma unroll
        for (int p = 0; p < PASSES; p++) {
            const int t = tid + NTH * p;
            const int m = t & 15, gi = t >> 4;          // row, group of 8 blocks
            const bool ok = m < M && 8 * gi < nb;
            const int mc = min(m, M - 1), gc = min(gi, nb / 8 - 1);
            const u32x4 dv = *reinterpret_cast<const u32x4*>(d + (int64_t)mc * nb + 8 * gc);
            const u32x4 s0 = *reinterpret_cast<const u32x4*>(s + (int64_t)mc * nb + 8 * gc);
            const u32x4 s1 = *reinterpret_cast<const u32x4*>(s + (int64_t)mc * nb + 8 * gc + 4);
            if (8 * gi < nb) {
                const uint32_t dw[4] = {dv.x, dv.y, dv.z, dv.w};
                const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const float f = ok ? h2f((dw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) : 0.0f;
                    dxl[(8 * gi + e) * 16 + m] = f;
                    dxsl[(8 * gi + e) * 16 + m] = ok ? f * (float)(int32_t)sw[e] : 0.0f;
                }
            }
        }
    }

    // A operands of the slice: activation row n16, K quarter g of each
    // block (rows past M and super-blocks past the slice: zero codes)
    u32x2 A[NST][NSP][8];
    {
        const int m = min(n16, M - 1);
#pragma unroll
        for (int st = 0; st < NST; st++)
#pragma unroll
            for (int h = 0; h < NSP; h++) {
                const int sb = sb0 + NSP * st + h;
                const bool ok = n16 < M && sb < sb1;
                const int sbc = min(sb, nsb - 1);
#pragma unroll
                for (int jj = 0; jj < 8; jj++) {
                    const u32x2 v = *reinterpret_cast<const u32x2*>(
                        q + (int64_t)m * Kp + 256 * sbc + 32 * jj + 8 * g);
                    A[st][h][jj] = ok ? v : u32x2{0u, 0u};
                }
            }
    }

    // global address and LDS offset of this lane's k-th chunk of item it
    auto chunk = [&](int it, int k, int& lo) {
        const int kt = it / NST, st = it - kt * NST;
        const int tile = b + kt * G;
        const int c = min(lane + 64 * k, TCH - 1);
        const int r = c / NCH, ch = c - r * NCH;
        const int row = min(16 * tile + r, N - 1);
        const int sb = min(sb0 + NSP * st + ch / 9, nsb - 1);
        lo = r * WSTR + 16 * ch;
        return w + (int64_t)row * row_bytes + (int64_t)sb * SBB + 16 * (ch % 9);
    };
    auto load_item = [&](int it, u32x4 (&R)[LPT]) {
        const int itc = min(it, nit - 1);
#pragma unroll
        for (int k = 0; k < LPT; k++) {
            int lo;
            R[k] = ld16_stream<true>(chunk(itc, k, lo));
        }
    };
    uint8_t* const mybuf = wbuf + wave * WBUF;
    auto commit = [&](int it, const u32x4 (&R)[LPT]) {
        const int itc = min(it, nit - 1);
#pragma unroll
        for (int k = 0; k < LPT; k++) {
            int lo;
            (void)chunk(itc, k, lo);
            st16(mybuf + lo, R[k]);
        }
        wave_sync();
    };

    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
    const i32x4 zero = {0, 0, 0, 0};

    int tile_now = 0;   // the tile whose stage compute() works on
    // the MFMAs and epilogue of stage st of the current tile (in mybuf)
    auto compute = [&](auto STc) {
        constexpr int st = decltype(STc)::value;
#pragma unroll
        for (int h = 0; h < NSP; h++) {
            const int sb = sb0 + NSP * st + h;
            const bool ok = sb < sb1;
            const int sbc = min(sb, nsb - 1);
            const uint8_t* rb = mybuf + n16 * WSTR + SBB * h;
            const u32x4 hdr = *reinterpret_cast<const u32x4*>(rb);
            const float fd = ok ? h2f(hdr.x & 0xFFFFu) : 0.0f;
            const float fdm = ok ? h2f(hdr.x >> 16) : 0.0f;
            const uint32_t slo = hdr.y & 0x3F3F3F3Fu;
            const uint32_t shi = (hdr.w & LO4) | ((hdr.y >> 2) & 0x30303030u);
            const uint32_t mlo = hdr.z & 0x3F3F3F3Fu;
            const uint32_t mhi = ((hdr.w >> 4) & LO4) | ((hdr.z >> 2) & 0x30303030u);
            const float* dxb = dxl + 8 * 16 * sbc;
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const u32x2 v = *reinterpret_cast<const u32x2*>(rb + 16 + 32 * c + 8 * g);
#pragma unroll
                for (int e = 0; e < 2; e++) {
                    const int jj = 2 * c + e;
                    const u32x2 bv = e == 0 ? u32x2{v.x & LO4, v.y & LO4}
                                            : u32x2{(v.x >> 4) & LO4, (v.y >> 4) & LO4};
                    const long Bo = (long)(((uint64_t)bv.y << 32) | bv.x);
                    const long Ao = (long)(((uint64_t)A[st][h][jj].y << 32) | A[st][h][jj].x);
                    const i32x4 D = __builtin_amdgcn_mfma_i32_16x16x32_i8(Ao, Bo, zero, 0, 0, 0);
                    if constexpr (DOTS) {
                        const int n = 16 * tile_now + n16;
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            const int m = 4 * g + i;
                            if (ok && m < M && n < N)
                                dots[((int64_t)m * N + n) * nb + 8 * sbc + jj] = D[i];
                        }
                    }
                    const float ws =
                        fd * (float)((((jj < 4 ? slo : shi) >> (8 * (jj & 3))) & 0xFFu));
                    const f32x4 x4 = *reinterpret_cast<const f32x4*>(dxb + 16 * jj + 4 * g);
#pragma unroll
                    for (int i = 0; i < 4; i++) acc[i] = fmaf((float)D[i], ws * x4[i], acc[i]);
                }
            }
            // min term: K lane g of block group kk is block 4 kk + g
#pragma unroll
            for (int kk = 0; kk < 2; kk++) {
                const float a = dxsl[16 * (8 * sbc + 4 * kk + g) + n16];
                const float bm = fdm * (float)bfe(kk ? mhi : mlo, 8 * g, 8);
                acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bm, acc2, 0, 0, 0);
            }
        }
    };

    lds_barrier();   // the scales are in LDS

    // DEPTH register sets hold the stages in flight; item it is in set
    // it % DEPTH.  Items go in rounds of DEPTH (TPR tiles of NST stages, all
    // unrolled, no branch around a load), the round past the last tile
    // running on clamped addresses with nothing stored.
    constexpr int TPR = DEPTH / NST > 0 ? DEPTH / NST : 1;   // tiles per round
    static_assert(NST % DEPTH == 0 || DEPTH % NST == 0, "rounds of whole tiles");
    // (the prologue issues the sets in item order and nothing after them:
    // the wait counts the compiler places at the loop head assume that
    // order, and an interleaved prologue makes it wait for every load there)
    u32x4 R[DEPTH][LPT];
    __builtin_amdgcn_sched_barrier(0);
    static_for<DEPTH>([&](auto Dc) {
        load_item(decltype(Dc)::value, R[decltype(Dc)::value]);
        __builtin_amdgcn_sched_barrier(0);
    });
    auto do_tile = [&](int kt, auto PARc) {
        constexpr int PAR = decltype(PARc)::value;
        static_for<NST>([&](auto STc) {
            constexpr int st = decltype(STc)::value;
            constexpr int set = (PAR + st) % DEPTH;
            const int it = kt * NST + st;
            tile_now = b + kt * G;
            commit(it, R[set]);
            load_item(it + DEPTH, R[set]);
            __builtin_amdgcn_sched_barrier(0);
            compute(STc);
            wave_sync();   // the buffer is read before the next commit
        });
        // the tile's partial sums meet in LDS; slice order is fixed
        float* sl = slot[kt & 1];
#pragma unroll
        for (int i = 0; i < 4; i++) sl[wave * 256 + (4 * g + i) * 16 + n16] = acc[i] - acc2[i];
        acc = f32x4{0.f, 0.f, 0.f, 0.f};
        acc2 = f32x4{0.f, 0.f, 0.f, 0.f};
        lds_barrier();
        if (tid < 256) {
            const int m = tid >> 4, n = 16 * (b + kt * G) + (tid & 15);
            float v = sl[tid];
#pragma unroll
            for (int ww = 1; ww < NW; ww++) v += sl[ww * 256 + tid];
            if (m < M && n < N) y[(int64_t)m * N + n] = v;
        }
    };
    for (int kt = 0; kt < ntk; kt += TPR) {
        static_for<TPR>([&](auto Tc) {
            constexpr int tt = decltype(Tc)::value;
            do_tile(kt + tt, std::integral_constant<int, (tt * NST) % DEPTH>{});
        });
    }
}

template <int NST, bool DOTS>
hipError_t launch_q4k(const void* w, int64_t N, int64_t K, int64_t M, const int8_t* q,
                      const uint16_t* d, const int32_t* s, float* y, int32_t* dots,
                      hipStream_t st) {
    const int Kp = (int)((K + 255) / 256 * 256);
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0) {
        (void)hipGetLastError();
        cus = 256;
    }
    const int64_t ntiles = (N + 15) / 16;
    const int64_t grid = ntiles < cus ? ntiles : cus;
    launch_kernel(k_sm3_q4k<NST, DOTS>, dim3((unsigned)grid), dim3(NTH), 0, st,
                  (const uint8_t*)w, (int)N, Kp, (int)M, q, d, s, y, dots);
    return hipGetLastError();
}

}  // namespace sm3

bool small_m3_supported(int fmt, int64_t K, int64_t M) {
    if (fmt != QGEMV_FMT_Q4_K || M < 1 || M > 16) return false;
    const int64_t nsb = (K + 255) / 256;
    const int64_t spw = (nsb + sm3::NW - 1) / sm3::NW;
    return spw <= 8 * sm3::NSP;
}

template <bool DOTS>
static hipError_t launch_m3(const void* w, int64_t N, int64_t K, int64_t M, const int8_t* q,
                            const uint16_t* d, const int32_t* s, float* y, int32_t* dots,
                            hipStream_t st) {
    const int64_t nsb = (K + 255) / 256;
    const int64_t spw = (nsb + sm3::NW - 1) / sm3::NW;
    const int64_t nst = (spw + sm3::NSP - 1) / sm3::NSP;
    // an even number of stages (a slice's stages past its super-blocks add
    // zeros)
    if (nst <= 2) return sm3::launch_q4k<2, DOTS>(w, N, K, M, q, d, s, y, dots, st);
    if (nst <= 4) return sm3::launch_q4k<4, DOTS>(w, N, K, M, q, d, s, y, dots, st);
    return sm3::launch_q4k<8, DOTS>(w, N, K, M, q, d, s, y, dots, st);
}

hipError_t launch_small_m3(int fmt, const void* w, int64_t N, int64_t K, int64_t M,
                           const int8_t* q, const uint16_t* d, const int32_t* s, float* y,
                           hipStream_t st) {
    if (!small_m3_supported(fmt, K, M)) return hipErrorNotSupported;
    return launch_m3<false>(w, N, K, M, q, d, s, y, nullptr, st);
}

hipError_t launch_small_m3_dots(int fmt, const void* w, int64_t N, int64_t K, int64_t M,
                                const int8_t* q, const uint16_t* d, const int32_t* s, float* y,
                                int32_t* dots, hipStream_t st) {
    if (!small_m3_supported(fmt, K, M)) return hipErrorNotSupported;
    return launch_m3<true>(w, N, K, M, q, d, s, y, dots, st);
}

}  // namespace qgemv
