// qgemv_quant.h -- the activation block quantiser and the SwiGLU product,
// shared by the quantisation kernels and the fused gate|up epilogue so that
// both produce the same bits.
//
// Per block of 32 ("Backends and hardware", section "CPU": the activation is
// quantised to int8 once per matmul): amax = max|x|; d32 = amax / 127 with an
// IEEE fp32 division; q = clamp(round_half_away(x / d32), -127, 127) with an
// IEEE division; d = fp16(d32) round-to-nearest-even; s = sum q.  All-zero
// blocks give d = 0, q = 0, s = 0.  Translation units including this file
// must be compiled without fast-math so that "/" is correctly rounded and
// roundf rounds half away from zero.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace qgemv {

// The lane's 4 codes packed in a dword; the block's fp16 scale bits and code
// sum, returned to every lane of the block.
struct QBlock {
    uint32_t packed;
    uint32_t dbits;
    int32_t sum;
};

// One block of 32 over 8 lanes, 4 consecutive values per lane; the block's 8
// lanes are an aligned group of 8 and all active.  Max and sum are reduced
// across the 8 lanes with cross-lane shuffles.
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

// SwiGLU: silu(g) * u with silu(g) = g / (1 + exp(-g)), in fp32.
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g / (1.0f + expf(-g)) * u;
}

}  // namespace qgemv
