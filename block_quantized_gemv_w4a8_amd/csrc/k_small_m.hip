// k_small_m.hip -- a few activation rows (the prefill chunk) against Q4_K
// weights.  Output row m equals the batch-1 GEMV of activation row m (colibri
// GPU backends, eligibility gates: C = A x B is row-independent).
//
// DOT4 variant: the GEMV kernel's mapping (LPR lanes per weight row, one
// 64-weight unit per lane step), except that each weight unit is loaded and
// unpacked once and then dotted against MT activation rows staged in LDS, so
// the weight stream is shared by the MT rows ("Backends and hardware",
// section "CUDA": W4A8 inner product on 4 x int8 dots).
#include "qgemv_device.h"
#include "qgemv_launch.h"

namespace qgemv {

constexpr int SWG = 256;

// LDS per activation row: Kp codes + fp32 dx[nb] + fp32 dx*s[nb].
__host__ __device__ inline int small_m_row_smem(int Kp) { return Kp + 8 * (Kp / 32); }

template <int MT, int LPR>
__global__ __launch_bounds__(SWG) void k_small_m_dot4(const uint8_t* __restrict__ w, int N,
                                                      int Kp, int U, int row_bytes, int M,
                                                      const int8_t* __restrict__ q,
                                                      const uint16_t* __restrict__ d,
                                                      const int32_t* __restrict__ s,
                                                      float* __restrict__ y, int R) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int nb = Kp / 32;
    const int m0 = blockIdx.y * MT;
    const int mc = min(MT, M - m0);
    const int rs = small_m_row_smem(Kp);
    const int tid = threadIdx.x;
    // stage the tile's activation rows
    for (int m = 0; m < mc; m++) {
        uint8_t* base = smem + m * rs;
        const int8_t* qm = q + (int64_t)(m0 + m) * Kp;
        for (int i = tid; i < Kp / 16; i += SWG)
            reinterpret_cast<u32x4*>(base)[i] = reinterpret_cast<const u32x4*>(qm)[i];
        float* dx = reinterpret_cast<float*>(base + Kp);
        for (int b = tid; b < nb; b += SWG) {
            const float f = h2f(d[(int64_t)(m0 + m) * nb + b]);
            dx[b] = f;
            dx[nb + b] = f * (float)s[(int64_t)(m0 + m) * nb + b];
        }
    }
    __syncthreads();

    constexpr int RPW = 64 / LPR;
    const int lane = tid & 63, wave = tid >> 6;
    const int li = lane % LPR;
    const int64_t base_row = (int64_t)blockIdx.x * R * 4 * RPW + wave * RPW + lane / LPR;
    for (int it = 0; it < R; it++) {
        const int64_t row = base_row + (int64_t)it * 4 * RPW;
        float acc[MT];
#pragma unroll
        for (int m = 0; m < MT; m++) acc[m] = 0.0f;
        if (row < N) {
            const uint8_t* rp = w + row * (int64_t)row_bytes;
            for (int u = li; u < U; u += LPR) {
                Q4K::W wv;
                Q4K::load(rp, u, wv);
                Q4K::C cc;
                Q4K::unpack(wv, cc);
                const float fd = h2f(wv.hdr.x & 0xFFFFu), fdm = h2f(wv.hdr.x >> 16);
                const int c = u & 3;
                int sc0, mn0, sc1, mn1;
                Q4K::scale_min(wv, 2 * c, sc0, mn0);
                Q4K::scale_min(wv, 2 * c + 1, sc1, mn1);
                const float ws0 = fd * (float)sc0, ws1 = fd * (float)sc1;
                const float wm0 = fdm * (float)mn0, wm1 = fdm * (float)mn1;
#pragma unroll
                for (int m = 0; m < MT; m++) {
                    if (m < mc) {
                        const uint8_t* am = smem + m * rs;
                        const float* dx = reinterpret_cast<const float*>(am + Kp);
                        Act16 x;
                        const u32x4* p = reinterpret_cast<const u32x4*>(am + 64 * u);
#pragma unroll
                        for (int k = 0; k < 4; k++) {
                            const u32x4 v = p[k];
                            x.a[4 * k] = v.x;
                            x.a[4 * k + 1] = v.y;
                            x.a[4 * k + 2] = v.z;
                            x.a[4 * k + 3] = v.w;
                        }
                        int D[2];
                        Q4K::dots_c(cc, x, D);
                        float t = acc[m];
                        t = fmaf((float)D[0], ws0 * dx[2 * u], t);
                        t = fmaf(-wm0, dx[nb + 2 * u], t);
                        t = fmaf((float)D[1], ws1 * dx[2 * u + 1], t);
                        t = fmaf(-wm1, dx[nb + 2 * u + 1], t);
                        acc[m] = t;
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MT; m++) {
            float a = acc[m];
#pragma unroll
            for (int off = LPR / 2; off > 0; off >>= 1) a += __shfl_xor(a, off, LPR);
            if (li == 0 && row < N && m < mc) y[(int64_t)(m0 + m) * N + row] = a;
        }
    }
}

template <int MT, int LPR>
static hipError_t launch_dot4(const void* w, int64_t N, int64_t K, int64_t M, const int8_t* q,
                              const uint16_t* d, const int32_t* s, float* y, hipStream_t st) {
    const int Kp = (int)((K + 255) / 256 * 256);
    const int U = Kp / 64;
    constexpr int RPW = 64 / LPR;
    const int64_t passes = (N + 4 * RPW - 1) / (4 * RPW);
    int R = (int)(passes / 2048);
    if (R < 1) R = 1;
    if (R > 16) R = 16;
    const int64_t gx = (passes + R - 1) / R;
    const int64_t gy = (M + MT - 1) / MT;
    const int smem = MT * small_m_row_smem(Kp);
    hipLaunchKernelGGL((k_small_m_dot4<MT, LPR>), dim3((unsigned)gx, (unsigned)gy), dim3(SWG),
                       smem, st, (const uint8_t*)w, (int)N, Kp, U, Kp / 256 * 144, (int)M, q, d,
                       s, y, R);
    return hipGetLastError();
}

template <int MT>
static hipError_t launch_dot4_mt(const void* w, int64_t N, int64_t K, int64_t M,
                                 const int8_t* q, const uint16_t* d, const int32_t* s, float* y,
                                 hipStream_t st) {
    const int U = (int)((K + 255) / 256 * 4);
    if (U > 32) return launch_dot4<MT, 64>(w, N, K, M, q, d, s, y, st);
    if (U > 16) return launch_dot4<MT, 32>(w, N, K, M, q, d, s, y, st);
    if (U > 8) return launch_dot4<MT, 16>(w, N, K, M, q, d, s, y, st);
    return launch_dot4<MT, 8>(w, N, K, M, q, d, s, y, st);
}

// Activation rows per tile: as many as fit in 64 KB of LDS, at most 8.
static int dot4_tile_rows(int64_t K) {
    const int Kp = (int)((K + 255) / 256 * 256);
    const int per = small_m_row_smem(Kp);
    int mt = 65536 / per;
    return mt >= 8 ? 8 : mt >= 4 ? 4 : mt >= 2 ? 2 : 1;
}

hipError_t launch_small_m_q4k(const void* w, int64_t N, int64_t K, int64_t M, const int8_t* q,
                              const uint16_t* d, const int32_t* s, float* y, int variant,
                              hipStream_t st) {
    (void)variant;
    int mt = dot4_tile_rows(K);
    if (M < mt) mt = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8;
    switch (mt) {
    case 8: return launch_dot4_mt<8>(w, N, K, M, q, d, s, y, st);
    case 4: return launch_dot4_mt<4>(w, N, K, M, q, d, s, y, st);
    case 2: return launch_dot4_mt<2>(w, N, K, M, q, d, s, y, st);
    default: return launch_dot4_mt<1>(w, N, K, M, q, d, s, y, st);
    }
}

}  // namespace qgemv
