// k_quantize.hip -- activation quantisation to int8 blocks of 32, and the
// fused SwiGLU (silu(gate) * up) + quantisation used between the gate|up and
// down products.
//
// The block quantiser itself (qgemv_quant.h) maps one block of 32 to 8
// lanes, 4 consecutive values per lane.
#include "qgemv_device.h"
#include "qgemv_launch.h"
#include "qgemv_quant.h"

namespace qgemv {

constexpr int QWG = 256;

__global__ __launch_bounds__(QWG) void k_quantize_act(const float* __restrict__ x, int64_t M,
                                                      int64_t K, int64_t ldx, int64_t Kp,
                                                      int8_t* __restrict__ q,
                                                      uint16_t* __restrict__ d,
                                                      int32_t* __restrict__ s) {
    const int64_t nb = Kp / 32;
    const int64_t gt = (int64_t)blockIdx.x * QWG + threadIdx.x;
    const int64_t blk = gt >> 3;
    const int sub = (int)(gt & 7);
    const bool live = blk < M * nb;
    const int64_t m = live ? blk / nb : 0;
    const int64_t b = live ? blk % nb : 0;
    const int64_t k0 = 32 * b + 4 * sub;
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; k++)
        v[k] = (live && k0 + k < K) ? x[m * ldx + k0 + k] : 0.0f;
    const QBlock r = quantize_block8(v);
    if (live) {
        *reinterpret_cast<uint32_t*>(q + m * Kp + k0) = r.packed;
        if (sub == 0) {
            d[m * nb + b] = (uint16_t)r.dbits;
            s[m * nb + b] = r.sum;
        }
    }
}

// h = silu(g) * u (fp32), then quantise h.
__global__ __launch_bounds__(QWG) void k_silu_mul_quantize(const float* __restrict__ gu,
                                                           int64_t N, int64_t Kp,
                                                           int8_t* __restrict__ q,
                                                           uint16_t* __restrict__ d,
                                                           int32_t* __restrict__ s,
                                                           float* __restrict__ h) {
    const int64_t nb = Kp / 32;
    const int64_t gt = (int64_t)blockIdx.x * QWG + threadIdx.x;
    const int64_t b = gt >> 3;
    const int sub = (int)(gt & 7);
    const bool live = b < nb;
    const int64_t k0 = 32 * b + 4 * sub;
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        float hv = 0.0f;
        if (live && k0 + k < N) {
            const float g = gu[k0 + k];
            const float u = gu[N + k0 + k];
            hv = silu_mul(g, u);
            if (h) h[k0 + k] = hv;
        }
        v[k] = hv;
    }
    const QBlock r = quantize_block8(v);
    if (live) {
        *reinterpret_cast<uint32_t*>(q + k0) = r.packed;
        if (sub == 0) {
            d[b] = (uint16_t)r.dbits;
            s[b] = r.sum;
        }
    }
}

hipError_t launch_quantize_act(const float* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                               uint16_t* d, int32_t* s, hipStream_t st) {
    const int64_t Kp = (K + 255) / 256 * 256;
    const int64_t threads = M * (Kp / 32) * 8;
    const int64_t grid = (threads + QWG - 1) / QWG;
    launch_kernel(k_quantize_act, dim3((unsigned)grid), dim3(QWG), 0, st, x, M, K, ldx, Kp,
                  q, d, s);
    return hipGetLastError();
}

hipError_t launch_silu_mul_quantize(const float* gu, int64_t N, int8_t* q, uint16_t* d,
                                    int32_t* s, float* h, hipStream_t st) {
    const int64_t Kp = (N + 255) / 256 * 256;
    const int64_t threads = (Kp / 32) * 8;
    const int64_t grid = (threads + QWG - 1) / QWG;
    launch_kernel(k_silu_mul_quantize, dim3((unsigned)grid), dim3(QWG), 0, st, gu, N, Kp, q,
                  d, s, h);
    return hipGetLastError();
}

}  // namespace qgemv
