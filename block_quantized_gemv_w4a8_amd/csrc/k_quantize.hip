// k_quantize.hip -- activation quantisation to int8 blocks of 32, and the
// fused SwiGLU (silu(gate) * up) + quantisation used between the gate|up and
// down products.
//
// The activation is quantised once per matmul ("Backends and hardware",
// section "CPU").  Per block of 32: amax = max|x|; d32 = amax / 127 with an
// IEEE fp32 division; q = clamp(round_half_away(x / d32), -127, 127) with an
// IEEE division; d = fp16(d32) round-to-nearest-even; s = sum q.  All-zero
// blocks give d = 0, q = 0, s = 0.  This file must be compiled without
// fast-math so that "/" is correctly rounded and roundf rounds half away.
//
// Mapping: 8 lanes per block, 4 consecutive values per lane; max and sum are
// reduced across the 8 lanes with cross-lane shuffles.
#include "qgemv_device.h"
#include "qgemv_launch.h"

namespace qgemv {

constexpr int QWG = 256;

// v: the lane's 4 values (the block's 8 lanes are aligned groups of 8).
// Returns the lane's 4 codes packed in a dword; the block's fp16 scale bits
// and code sum are returned to every lane of the block.
struct QBlock {
    uint32_t packed;
    uint32_t dbits;
    int32_t sum;
};

__device__ __forceinline__ QBlock quantize_block8(const float v[4]) {
    float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 8));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 8));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 8));
    uint32_t packed = 0;
    int sum = 0;
    float d32 = 0.0f;
    if (amax != 0.0f) {
        d32 = amax / 127.0f;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            float r = roundf(v[k] / d32);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            const int qi = (int)r;
            sum += qi;
            packed |= ((uint32_t)qi & 0xFFu) << (8 * k);
        }
    }
    sum += __shfl_xor(sum, 1, 8);
    sum += __shfl_xor(sum, 2, 8);
    sum += __shfl_xor(sum, 4, 8);
    return QBlock{packed, (uint32_t)__half_as_ushort(__float2half_rn(d32)), sum};
}

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

// h = silu(g) * u with silu(g) = g / (1 + exp(-g)), fp32; then quantise h.
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
            hv = g / (1.0f + expf(-g)) * u;
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
    hipLaunchKernelGGL(k_quantize_act, dim3((unsigned)grid), dim3(QWG), 0, st, x, M, K, ldx, Kp,
                       q, d, s);
    return hipGetLastError();
}

hipError_t launch_silu_mul_quantize(const float* gu, int64_t N, int8_t* q, uint16_t* d,
                                    int32_t* s, float* h, hipStream_t st) {
    const int64_t Kp = (N + 255) / 256 * 256;
    const int64_t threads = (Kp / 32) * 8;
    const int64_t grid = (threads + QWG - 1) / QWG;
    hipLaunchKernelGGL(k_silu_mul_quantize, dim3((unsigned)grid), dim3(QWG), 0, st, gu, N, Kp, q,
                       d, s, h);
    return hipGetLastError();
}

}  // namespace qgemv
