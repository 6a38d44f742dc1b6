// qgemv_quant.h -- the activation block quantiser and the SwiGLU product,
// shared by the quantisation kernels, the fused gate|up epilogue and the
// GEMVs that quantise their own input, so that all produce the same bits.
//
// Per block of 32 ("Backends and hardware", section "CPU": the activation is
// quantised to int8 once per matmul): amax = max|x|; d32 = amax / 127 with an
// IEEE fp32 division; q = clamp(round_half_away(x / d32), -127, 127) with the
// quotient correctly rounded to fp32; d = fp16(d32) round-to-nearest-even;
// s = sum q.  All-zero blocks give d = 0, q = 0, s = 0.  Translation units
// including this file must be compiled without fast-math so that "/" is
// correctly rounded and roundf rounds half away from zero.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace qgemv {

// A value from another lane of the same aligned group of L lanes (L = 2, 4
// or 8), by DPP (no LDS round trip): quad_perm [1,0,3,2], quad_perm
// [2,3,0,1], then the lane mirrored within the group of 8, which lies in the
// other quad.
template <int CTRL>
__device__ __forceinline__ int dpp_lane(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int L>
__device__ __forceinline__ float group_max(float v) {
    static_assert(L == 2 || L == 4 || L == 8, "groups of 2, 4 or 8 lanes");
    v = fmaxf(v, __builtin_bit_cast(float, dpp_lane<0xB1>(__builtin_bit_cast(int, v))));
    if constexpr (L >= 4)
        v = fmaxf(v, __builtin_bit_cast(float, dpp_lane<0x4E>(__builtin_bit_cast(int, v))));
    if constexpr (L >= 8)
        v = fmaxf(v, __builtin_bit_cast(float, dpp_lane<0x141>(__builtin_bit_cast(int, v))));
    return v;
}
template <int L>
__device__ __forceinline__ int group_isum(int v) {
    v += dpp_lane<0xB1>(v);
    if constexpr (L >= 4) v += dpp_lane<0x4E>(v);
    if constexpr (L >= 8) v += dpp_lane<0x141>(v);
    return v;
}

// The lane's 32/L codes packed in 8/L dwords (value i of the lane in byte
// i % 4 of dword i / 4); the block's fp16 scale bits and code sum, returned
// to every lane of the block.
template <int L>
struct QBlockL {
    uint32_t packed[8 / L];
    uint32_t dbits;
    int32_t sum;
};

// One block of 32 over L lanes (an aligned, fully active group), 32/L
// consecutive values per lane.  Max and sum are reduced across the L lanes
// (exact, so the lane count and order do not change any bit) and every lane
// of the group receives them.
template <int L>
__device__ __forceinline__ QBlockL<L> quantize_block(const float (&v)[32 / L]) {
#pragma clang fp contract(off)
    constexpr int V = 32 / L;
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < V; k++) amax = fmaxf(amax, fabsf(v[k]));
    amax = group_max<L>(amax);
    QBlockL<L> r;
#pragma unroll
    for (int k = 0; k < 8 / L; k++) r.packed[k] = 0u;
    int sum = 0;
    float d32 = 0.0f;
    if (amax != 0.0f) {
        d32 = amax / 127.0f;
        // x / d32 is formed as x * rcp with rcp within 1 ulp of 1 / d32: the
        // product is within 2^-22 relative -- at most 2^-15 absolute, as
        // |x / d32| <= 127.01 -- of the correctly rounded quotient, so both
        // round to the same integer unless the product lies within 2^-13 of a
        // boundary k + 1/2 (where rint's ties-to-even would also differ from
        // rounding half away).  Such a value (about one in 4096), or every
        // value of a block whose 1 / d32 would leave the normal range, is
        // divided instead.  A lane almost never holds two such values, so the
        // one it holds is selected, divided once and put back, in straight-
        // line code (taken branches around each value's division cost a wave
        // ~0.7 us); lanes with more go through every value.  Either way q is
        // the rounding of the correctly rounded quotient.
        constexpr float kBand = 0.5f - 0x1p-13f;
        const float rcp = __builtin_amdgcn_rcpf(d32);
        const bool ranged = d32 >= 0x1p-120f && d32 <= 0x1p120f;
        float qf[V], y[V];
        float far = 0.0f;   // largest distance to the nearest integer
#pragma unroll
        for (int k = 0; k < V; k++) {
            y[k] = v[k] * rcp;
            qf[k] = __builtin_rintf(y[k]);
            far = fmaxf(far, fabsf(y[k] - qf[k]));   // an exact difference
        }
        if (!ranged || far >= kBand) {
            bool f[V];
            int nflag = 0;
            float vs = 0.0f;
#pragma unroll
            for (int k = 0; k < V; k++) {
                f[k] = !ranged || fabsf(y[k] - qf[k]) >= kBand;
                nflag += f[k] ? 1 : 0;
                vs = f[k] ? v[k] : vs;
            }
            if (nflag == 1) {
                const float qd = roundf(vs / d32);
#pragma unroll
                for (int k = 0; k < V; k++) qf[k] = f[k] ? qd : qf[k];
            } else {
#pragma unroll
                for (int k = 0; k < V; k++)
                    if (f[k]) qf[k] = roundf(v[k] / d32);
            }
        }
#pragma unroll
        for (int k = 0; k < V; k++) {
            const int qi = (int)fminf(fmaxf(qf[k], -127.0f), 127.0f);
            sum += qi;
            r.packed[k / 4] |= ((uint32_t)qi & 0xFFu) << (8 * (k % 4));
        }
    }
    r.sum = group_isum<L>(sum);
    r.dbits = (uint32_t)__half_as_ushort(__float2half_rn(d32));
    return r;
}

// The 8-lane form (4 values per lane) used by the quantisation kernels.
struct QBlock {
    uint32_t packed;
    uint32_t dbits;
    int32_t sum;
};
__device__ __forceinline__ QBlock quantize_block8(const float (&v)[4]) {
    const QBlockL<8> r = quantize_block<8>(v);
    return QBlock{r.packed[0], r.dbits, r.sum};
}

// SwiGLU: silu(g) * u with silu(g) = g / (1 + exp(-g)), in fp32.
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g / (1.0f + expf(-g)) * u;
}

}  // namespace qgemv
