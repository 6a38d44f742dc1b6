// k_gemv.h -- batch-1 W4A8 GEMV kernels (Q4_0, Q4_K, Q6_K, Q8_0) and their
// launchers, as templates over the weight format.  Each format's launchers
// are instantiated in a translation unit of their own (k_gemv_<fmt>.hip,
// through QGEMV_GEMV_FORMAT_ENTRIES below); k_gemv.hip holds the dispatch by
// format, the Q6_K repack and the block-dots validation kernel.
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
#pragma once

#include <atomic>
#include <map>
#include <mutex>
#include <utility>

#include "qgemv_device.h"
#include "qgemv_launch.h"
#include "qgemv_quant.h"

namespace qgemv {

constexpr int WG = 256;  // 4 wavefronts of 64

// Sum over aligned groups of LPR lanes with DPP (no LDS round trip).  The
// total of each group is valid in the group's last lane (li == LPR - 1); the
// order of the additions is fixed, so results are deterministic.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float,
        __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
    v += dpp<0xB1, 0xF>(v);                        // quad_perm [1,0,3,2]
    v += dpp<0x4E, 0xF>(v);                        // quad_perm [2,3,0,1]
    if constexpr (LPR >= 8) v += dpp<0x141, 0xF>(v);   // row_half_mirror
    if constexpr (LPR >= 16) v += dpp<0x140, 0xF>(v);  // row_mirror
    if constexpr (LPR >= 32) v += dpp<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
    if constexpr (LPR >= 64) v += dpp<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
    return v;
}

// The activation of one unit, held in registers for the whole kernel: a lane
// always covers the same units of every row it visits.
template <int FMT>
struct ActReg;

template <>
struct ActReg<QGEMV_FMT_Q4_K> {
    Act16 x;
    float dx[2], dxs[2];  // blocks 2u, 2u+1: f(dx) and f(dx) * s (exact in fp32)
    __device__ void load(const int8_t* q, const uint16_t* d, const int32_t* s, int u) {
        const u32x4* p = reinterpret_cast<const u32x4*>(q + 64 * u);
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const u32x4 v = p[k];
            x.a[4 * k] = v.x; x.a[4 * k + 1] = v.y; x.a[4 * k + 2] = v.z; x.a[4 * k + 3] = v.w;
        }
#pragma unroll
        for (int jj = 0; jj < 2; jj++) {
            dx[jj] = h2f(d[2 * u + jj]);
            dxs[jj] = dx[jj] * (float)s[2 * u + jj];
        }
    }
};

template <>
struct ActReg<QGEMV_FMT_Q6_K> {
    Act16 x;
    float dx[4];
    int init[4];  // -32 * (sum of the group's 16 codes)
    __device__ void load(const int8_t* q, const uint16_t* d, const int32_t*, int u) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int off = Q6K::act_offset(u, j);
            const u32x4 v = *reinterpret_cast<const u32x4*>(q + off);
            x.a[4 * j] = v.x; x.a[4 * j + 1] = v.y; x.a[4 * j + 2] = v.z; x.a[4 * j + 3] = v.w;
            init[j] = -32 * sum16(v.x, v.y, v.z, v.w);
            dx[j] = h2f(d[off >> 5]);
        }
    }
};

template <>
struct ActReg<QGEMV_FMT_Q6_K_R8> : ActReg<QGEMV_FMT_Q6_K> {};

template <>
struct ActReg<QGEMV_FMT_Q4_0> {
    Act16 x;
    float dx[2];
    int init[2];  // -8 * s_b
    __device__ void load(const int8_t* q, const uint16_t* d, const int32_t* s, int u) {
        const u32x4* p = reinterpret_cast<const u32x4*>(q + 64 * u);
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const u32x4 v = p[k];
            x.a[4 * k] = v.x; x.a[4 * k + 1] = v.y; x.a[4 * k + 2] = v.z; x.a[4 * k + 3] = v.w;
        }
#pragma unroll
        for (int jj = 0; jj < 2; jj++) {
            dx[jj] = h2f(d[2 * u + jj]);
            init[jj] = -8 * s[2 * u + jj];
        }
    }
};

template <>
struct ActReg<QGEMV_FMT_Q8_0> {
    Act16 x;
    float dx[2];
    __device__ void load(const int8_t* q, const uint16_t* d, const int32_t*, int u) {
        const u32x4* p = reinterpret_cast<const u32x4*>(q + 64 * u);
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const u32x4 v = p[k];
            x.a[4 * k] = v.x; x.a[4 * k + 1] = v.y; x.a[4 * k + 2] = v.z; x.a[4 * k + 3] = v.w;
        }
        dx[0] = h2f(d[2 * u]);
        dx[1] = h2f(d[2 * u + 1]);
    }
};

// An fp32 activation row quantised by the whole workgroup into LDS: codes
// aq [Kp], fp16 scale bits ad [Kp/32] and code sums as [Kp/32], blocks past K
// zero.  The block quantiser is the one of k_quantize_act with XqLanes<NTH>
// lanes per block of 32 (2 for 256 threads, 4 for 512: 16 or 8 consecutive
// values each) instead of 8: max and sum are exact, so the bits are the
// same, and the per-block work (max, scale, sum) is shared by the lane's
// values.  One pass covers NTH / XqLanes blocks (128 at both sizes, so every
// thread has values at K = 4096); each load's address is clamped into x and
// lane parts past K are masked to zero.  The first pass's loads are issued by
// the caller (xq_load) ahead of its weight loads.
template <int NTH>
constexpr int XqLanes = NTH >= 512 ? 4 : 2;
template <int NTH>
constexpr int XqLoads = 32 / XqLanes<NTH> / 4;   // f32x4 loads per lane and pass

template <int NTH = WG>
__device__ __forceinline__ void xq_load(const float* __restrict__ x, int K, int b0,
                                        f32x4 (&v)[XqLoads<NTH>]) {
    constexpr int L = XqLanes<NTH>;
    const int e = 32 * (b0 + (int)threadIdx.x / L) + (32 / L) * ((int)threadIdx.x % L);
#pragma unroll
    for (int k = 0; k < XqLoads<NTH>; k++)
        v[k] = *reinterpret_cast<const f32x4*>(x + min(e + 4 * k, K - 4));
}

template <int NTH = WG>
__device__ __forceinline__ void xq_batch(const f32x4 (&v)[XqLoads<NTH>], int K, int nb, int b0,
                                         int8_t* aq, uint16_t* ad, int32_t* as) {
    constexpr int L = XqLanes<NTH>, V = 32 / L;
    const int b = b0 + (int)threadIdx.x / L, part = (int)threadIdx.x % L;
    const int e = 32 * b + V * part;
    const bool in = e < K;
    float vv[V];
#pragma unroll
    for (int k = 0; k < V / 4; k++) {
        vv[4 * k] = in ? v[k].x : 0.0f;
        vv[4 * k + 1] = in ? v[k].y : 0.0f;
        vv[4 * k + 2] = in ? v[k].z : 0.0f;
        vv[4 * k + 3] = in ? v[k].w : 0.0f;
    }
    const QBlockL<L> r = quantize_block<L>(vv);
    if (b < nb) {
        if constexpr (L == 2)
            *reinterpret_cast<u32x4*>(aq + e) =
                u32x4{r.packed[0], r.packed[1], r.packed[2], r.packed[3]};
        else
            *reinterpret_cast<uint2*>(aq + e) = uint2{r.packed[0], r.packed[1]};
        if (part == 0) {
            ad[b] = (uint16_t)r.dbits;
            as[b] = r.sum;
        }
    }
}

template <int NTH = WG>
__device__ __forceinline__ void quantize_row_lds(const float* __restrict__ x, int K, int Kp,
                                                 const f32x4 (&first)[XqLoads<NTH>], int8_t* aq,
                                                 uint16_t* ad, int32_t* as) {
    const int nb = Kp / 32;
    constexpr int BATCH = NTH / XqLanes<NTH>;   // blocks per pass
    xq_batch<NTH>(first, K, nb, 0, aq, ad, as);
    for (int b0 = BATCH; b0 < nb; b0 += BATCH) {
        f32x4 v[XqLoads<NTH>];
        xq_load<NTH>(x, K, b0, v);
        xq_batch<NTH>(v, K, nb, b0, aq, ad, as);
    }
}

// Workgroup 0 of a product that quantised x itself writes the codes out.
template <int NTH = WG>
__device__ __forceinline__ void xq_write_out(const ActIn& ai, int Kp, const int8_t* aq,
                                             const uint16_t* ad, const int32_t* as) {
    for (int t = threadIdx.x; t < Kp / 16; t += NTH)
        *reinterpret_cast<u32x4*>(ai.q + 16 * t) = *reinterpret_cast<const u32x4*>(aq + 16 * t);
    for (int t = threadIdx.x; t < Kp / 32; t += NTH) {
        ai.d[t] = ad[t];
        ai.s[t] = as[t];
    }
}

// Bytes of LDS an in-kernel quantised activation row takes (codes, fp16
// scales, int32 sums).
__host__ __device__ inline int act_lds_bytes(int Kp) { return Kp + Kp / 16 + Kp / 8; }

template <int FMT>
struct Unit;
template <>
struct Unit<QGEMV_FMT_Q4_K> {
    using W = Q4K::W;
    __device__ static void load(const uint8_t* rp, int u, bool, W& w) { Q4K::load(rp, u, w); }
    __device__ static float term(const W& w, const ActReg<QGEMV_FMT_Q4_K>& a, int u, int) {
        int D[2];
        Q4K::dots(w, a.x, D);
        const float fd = h2f(w.hdr.x & 0xFFFFu), fdm = h2f(w.hdr.x >> 16);
        const int c = u & 3;
        float t = 0.0f;
#pragma unroll
        for (int jj = 0; jj < 2; jj++) {
            int sc, mn;
            Q4K::scale_min(w, 2 * c + jj, sc, mn);
            t = fmaf((float)D[jj], fd * (float)sc * a.dx[jj], t);
            t = fmaf(-(fdm * (float)mn), a.dxs[jj], t);
        }
        return t;
    }
};
template <>
struct Unit<QGEMV_FMT_Q6_K> {
    using W = Q6K::W;
    __device__ static void load(const uint8_t* rp, int u, bool, W& w) { Q6K::load(rp, u, w); }
    __device__ static float term(const W& w, const ActReg<QGEMV_FMT_Q6_K>& a, int u, int) {
        int D[4];
        Q6K::dots(w, a.x, a.init, D);
        const float fd = h2f(w.d);
        float t = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; j++)
            t = fmaf((float)D[j], fd * (float)Q6K::scale(w, u, j) * a.dx[j], t);
        return t;
    }
};
template <>
struct Unit<QGEMV_FMT_Q6_K_R8> {
    using W = Q6K::W;
    __device__ static void load(const uint8_t* rp, int u, bool, W& w) { Q6K::load_r8(rp, u, w); }
    __device__ static float term(const W& w, const ActReg<QGEMV_FMT_Q6_K_R8>& a, int u, int nbw) {
        return Unit<QGEMV_FMT_Q6_K>::term(w, a, u, nbw);
    }
};
template <>
struct Unit<QGEMV_FMT_Q4_0> {
    using W = Q40::W;
    __device__ static void load(const uint8_t* rp, int u, bool has1, W& w) {
        Q40::load(rp, u, has1, w);
    }
    __device__ static float term(const W& w, const ActReg<QGEMV_FMT_Q4_0>& a, int, int) {
        int D[2];
        Q40::dots(w, a.x, a.init, D);
        // a missing second block has d1 = 0, so its term is exactly zero
        return fmaf((float)D[1], h2f(w.d1) * a.dx[1], (float)D[0] * (h2f(w.d0) * a.dx[0]));
    }
};
template <>
struct Unit<QGEMV_FMT_Q8_0> {
    using W = Q80::W;
    __device__ static void load(const uint8_t* rp, int u, bool has1, W& w) {
        Q80::load(rp, u, has1, w);
    }
    __device__ static float term(const W& w, const ActReg<QGEMV_FMT_Q8_0>& a, int, int) {
        int D[2];
        Q80::dots(w, a.x, D);
        return fmaf((float)D[1], h2f(w.d1) * a.dx[1], (float)D[0] * (h2f(w.d0) * a.dx[0]));
    }
};

constexpr int SEGP = 64;  // passes whose split-K partial sums are buffered in LDS

// Persistent GEMV.  The grid is sized to the number of workgroups that fit
// on the chip at once.  The rows are cut into groups of RPP consecutive rows
// (one group per workgroup pass) and the groups are dealt round-robin over the
// workgroups, so at any moment the whole chip streams one contiguous window of
// the weight matrix (measured faster on MI355X than giving each workgroup a
// contiguous slab).  Inside a workgroup the 4 waves form 4/WK row groups; the
// WK waves of a group split the row's units into WK contiguous slices
// (split-K for long rows) whose partial sums meet in LDS.  Lane li of a wave
// covers the units u = slice_start + li + LPR*i (i < UPL) of every row it
// visits, so its activation lives in registers for the whole kernel.  Two row
// buffers are used in turn: the next row's loads are in flight while the
// current row is computed.
// Rows of this kernel that quantise their own activation (XQ) are at most
// this long (the LDS-streaming kernel takes longer ones).
constexpr int kXqShortKp = 2048;

// MULTI: the rows are those of several matrices (mr), each with its own
// weights and output; row r of the combined range is row r - start[m] of
// matrix m (selected without indexing the argument arrays by lane).
template <int FMT, int LPR, int UPL, int WK, bool XQ, bool MULTI>
__global__ __launch_bounds__(WG) void k_gemv(const uint8_t* __restrict__ w, int N, int U,
                                              int US, int nbw, int row_bytes,
                                              const int8_t* __restrict__ q,
                                              const uint16_t* __restrict__ d,
                                              const int32_t* __restrict__ s,
                                              float* __restrict__ y, const ActIn ai,
                                              const MultiRows mr) {
    static_assert(WK == 1 || LPR == 64, "split-K needs whole waves per row");
    static_assert(!MULTI || WK == 1, "several matrices: whole rows per lane group");
    // matrix m of combined row r, its row pointer and output
    auto mat_of = [&](int64_t r) {
        int m = 0;
#pragma unroll
        for (int k = 1; k < kMultiMax; k++) m += (k < mr.count && r >= mr.start[k]) ? 1 : 0;
        return m;
    };
    auto row_ptr = [&](int64_t r) -> const uint8_t* {
        if constexpr (!MULTI) return w + r * (int64_t)row_bytes;
        const int m = mat_of(r);
        const uint8_t* base = static_cast<const uint8_t*>(mr.w[0]);
        int start = mr.start[0];
#pragma unroll
        for (int k = 1; k < kMultiMax; k++) {
            base = m == k ? static_cast<const uint8_t*>(mr.w[k]) : base;
            start = m == k ? mr.start[k] : start;
        }
        return base + (r - start) * (int64_t)row_bytes;
    };
    auto out_ptr = [&](int64_t r) -> float* {
        if constexpr (!MULTI) return y + r;
        const int m = mat_of(r);
        float* base = mr.y[0];
        int start = mr.start[0];
#pragma unroll
        for (int k = 1; k < kMultiMax; k++) {
            base = m == k ? mr.y[k] : base;
            start = m == k ? mr.start[k] : start;
        }
        return base + (r - start);
    };
    constexpr int RPW = 64 / LPR;
    constexpr int NRG = 4 / WK;
    constexpr int RPP = NRG * RPW;  // rows per workgroup pass (one row group)
    __shared__ float part[WK > 1 ? SEGP * RPP * WK : 1];
    using UnitT = Unit<FMT>;
    using WT = typename UnitT::W;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kq = wave % WK, rg = wave / WK;
    const int li = lane % LPR, sub = lane / LPR;
    const int u_lo = kq * US;
    const int u_hi = min(U, u_lo + US);

    // Lanes past the end of their slice repeat the slice's last unit (so every
    // load is unconditional and in bounds) and drop its contribution.
    ActReg<FMT> A[UPL];
    int uu[UPL];
    bool ok[UPL];
#pragma unroll
    for (int i = 0; i < UPL; i++) {
        const int u = u_lo + li + LPR * i;
        ok[i] = u < u_hi;
        uu[i] = ok[i] ? u : u_hi - 1;
        if constexpr (!XQ) A[i].load(q, d, s, uu[i]);
    }
    // XQ: the activation row quantised in this workgroup (codes, fp16
    // scales, sums; Kp <= kXqShortKp)
    __shared__ __align__(16) uint8_t xq_lds[XQ ? kXqShortKp + kXqShortKp / 16 + kXqShortKp / 8 : 16];
    const int Kp = (32 * nbw + 255) / 256 * 256;
    int8_t* const aq = reinterpret_cast<int8_t*>(xq_lds);
    uint16_t* const ad = reinterpret_cast<uint16_t*>(xq_lds + Kp);
    int32_t* const as = reinterpret_cast<int32_t*>(xq_lds + Kp + Kp / 16);

    const int my_off = rg * RPW + sub;  // this lane's row within a group
    const int64_t G = gridDim.x;
    const int64_t ngroups = ((int64_t)N + RPP - 1) / RPP;
    // row of pass p (passes counted from this workgroup's first group)
    auto row_of = [&](int64_t p) { return (blockIdx.x + p * G) * RPP + my_off; };
    // Rows past N reload row N-1: loads never sit under a lane-dependent
    // branch, so the compiler waits for exactly the loads a row needs while
    // the next row's loads stay in flight.
    auto load_row = [&](WT (&wv)[UPL], int64_t row) {
        const uint8_t* rp = row_ptr(min(row, (int64_t)N - 1));
#pragma unroll
        for (int i = 0; i < UPL; i++) UnitT::load(rp, uu[i], 2 * uu[i] + 1 < nbw, wv[i]);
    };
    // Dot one loaded row and reduce it over the row's lanes; the row sum (or
    // this wave's split-K part of it) is valid in lane li == LPR - 1.
    auto dot_row = [&](const WT (&wv)[UPL]) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < UPL; i++) {
            const float t = UnitT::term(wv[i], A[i], uu[i], nbw);
            acc += ok[i] ? t : 0.0f;
        }
        return group_sum<LPR>(acc);
    };
    auto finish_row = [&](float acc, int64_t row, int pl) {
        if (li == LPR - 1 && row < N) {
            if constexpr (WK == 1) *out_ptr(row) = acc;
            else part[(pl * RPP + my_off) * WK + kq] = acc;
        }
    };

    const int64_t npass_all = ngroups > (int64_t)blockIdx.x
                                  ? (ngroups - blockIdx.x + G - 1) / G : 0;
    // The first row's loads go out before anything waits for the
    // activation's, so the weight stream starts one load latency sooner; a
    // segment's last pass loads the next segment's first row into wa (SEGP
    // is even).
    static_assert(SEGP % 2 == 0, "segments of whole row pairs");
    WT wa[UPL], wb[UPL];
    load_row(wa, row_of(0));
    __builtin_amdgcn_sched_barrier(0);
    for (int64_t p0 = 0; p0 < npass_all; p0 += SEGP) {
        const int np = (int)min((int64_t)SEGP, npass_all - p0);
        if constexpr (XQ) {
            if (p0 == 0) {
                // the first row's weights are on their way; quantise x
                f32x4 xv[XqLoads<WG>];
                xq_load(ai.x, 32 * nbw, 0, xv);
                quantize_row_lds(ai.x, 32 * nbw, Kp, xv, aq, ad, as);
                __syncthreads();
#pragma unroll
                for (int i = 0; i < UPL; i++) A[i].load(aq, ad, as, uu[i]);
                if (blockIdx.x == 0) {
                    for (int t = threadIdx.x; t < Kp / 16; t += WG)
                        *reinterpret_cast<u32x4*>(ai.q + 16 * t) =
                            *reinterpret_cast<const u32x4*>(aq + 16 * t);
                    for (int t = threadIdx.x; t < Kp / 32; t += WG) {
                        ai.d[t] = ad[t];
                        ai.s[t] = as[t];
                    }
                }
            }
        }
        // (sched_barrier keeps the compiler from sinking a row's loads below
        // the wait for the previous row.)
        for (int p = 0; p < np; p += 2) {
            load_row(wb, row_of(p0 + p + 1));
            __builtin_amdgcn_sched_barrier(0);
            finish_row(dot_row(wa), row_of(p0 + p), p);
            load_row(wa, row_of(p0 + p + 2));
            __builtin_amdgcn_sched_barrier(0);
            if (p + 1 < np) finish_row(dot_row(wb), row_of(p0 + p + 1), p + 1);
        }
        if constexpr (WK > 1) {
            __syncthreads();
            for (int t = threadIdx.x; t < np * RPP; t += WG) {
                const int64_t row = (blockIdx.x + (p0 + t / RPP) * G) * RPP + t % RPP;
                if (row < N) {
                    float v = part[t * WK];
#pragma unroll
                    for (int k = 1; k < WK; k++) v += part[t * WK + k];
                    y[row] = v;
                }
            }
            __syncthreads();
        }
    }
}

// Unit loaders for the LDS-streaming kernel.  The slice of a row sits in LDS
// in its original byte order, starting `off0` bytes into the buffer (the
// chunk grid is aligned to 16-byte global addresses, see k_gemv_lds).  Q4_K
// fields are 16-byte aligned there; Q6_K, Q4_0 and Q8_0 blocks start every
// 210, 18 or 34 bytes, so their fields can sit 2 bytes off a 4-byte boundary.
// Those are read as aligned dwords and shifted into place with v_alignbyte
// (lds16_a2, lds8_a2 in qgemv_device.h).
template <int FMT>
struct UnitLds;
template <>
struct UnitLds<QGEMV_FMT_Q4_K> {
    static constexpr int UNITS_PER_BLK = 4, BLK_BYTES = 144;
    // (super-blocks are 144 = 9 x 16 bytes: the slice always starts aligned)
    __device__ static void load(const uint8_t* b, int off0, int ul, bool, Q4K::W& w) {
        const int p = off0 + 144 * (ul >> 2);
        const int c = ul & 3;
        w.hdr = lds16(b, p);
        w.qa = lds16(b, p + 16 + 32 * c);
        w.qb = lds16(b, p + 32 + 32 * c);
    }
};
template <>
struct UnitLds<QGEMV_FMT_Q6_K> {
    static constexpr int UNITS_PER_BLK = 4, BLK_BYTES = 210;
    __device__ static void load(const uint8_t* b, int off0, int ul, bool, Q6K::W& w) {
        const int p = off0 + 210 * (ul >> 2);
        const int h = (ul >> 1) & 1, t = ul & 1;
        w.qa = lds16_a2(b, p + 64 * h + 16 * t);
        w.qb = lds16_a2(b, p + 64 * h + 32 + 16 * t);
        w.qh = lds16_a2(b, p + 128 + 32 * h + 16 * t);
        w.sc = lds8_a2(b, p + 192 + 8 * h);
        w.d = lds2(b, p + 208);
    }
};
template <>
struct UnitLds<QGEMV_FMT_Q6_K_R8> {
    // slices start at tile boundaries, so off0 is a multiple of 16 and every
    // field is read with one aligned LDS access
    __device__ static void load(const uint8_t* b, int off0, int ul, bool, Q6K::W& w) {
        const int S = ul >> 2, i = S & 7;
        const int p = off0 + Q6K::TILE_BYTES * (S >> 3);
        const int h = (ul >> 1) & 1, t = ul & 1;
        w.qa = lds16(b, p + 128 * i + 64 * h + 16 * t);
        w.qb = lds16(b, p + 128 * i + 64 * h + 32 + 16 * t);
        w.qh = lds16(b, p + Q6K::T_QH + 64 * i + 32 * h + 16 * t);
        w.sc = *reinterpret_cast<const u32x2*>(b + p + Q6K::T_SC + 16 * i + 8 * h);
        w.d = lds2(b, p + Q6K::T_D + 2 * i);
    }
};
template <>
struct UnitLds<QGEMV_FMT_Q4_0> {
    static constexpr int UNITS_PER_BLK = 0, BLK_BYTES = 18;
    // a missing second block re-reads the first one and gets d1 = 0
    __device__ static void load(const uint8_t* b, int off0, int ul, bool has1, Q40::W& w) {
        const int p0 = off0 + 36 * ul;
        const int p1 = has1 ? p0 + 18 : p0;
        w.d0 = lds2(b, p0);
        w.q0 = lds16_a2(b, p0 + 2);
        const uint32_t d1 = lds2(b, p1);
        w.d1 = has1 ? d1 : 0u;
        w.q1 = lds16_a2(b, p1 + 2);
    }
};
template <>
struct UnitLds<QGEMV_FMT_Q8_0> {
    static constexpr int UNITS_PER_BLK = 0, BLK_BYTES = 34;
    __device__ static void load(const uint8_t* b, int off0, int ul, bool has1, Q80::W& w) {
        const int p0 = off0 + 68 * ul;
        const int p1 = has1 ? p0 + 34 : p0;
        w.d0 = lds2(b, p0);
        w.a0 = lds16_a2(b, p0 + 2);
        w.b0 = lds16_a2(b, p0 + 18);
        const uint32_t d1 = lds2(b, p1);
        w.d1 = has1 ? d1 : 0u;
        w.a1 = lds16_a2(b, p1 + 2);
        w.b1 = lds16_a2(b, p1 + 18);
    }
};

// Byte offset of unit u within a row, and the first block of unit u.
template <int FMT>
__host__ __device__ inline int unit_byte(int u) {
    if (FMT == QGEMV_FMT_Q4_K) return (u / 4) * 144;
    if (FMT == QGEMV_FMT_Q6_K) return (u / 4) * 210;
    if (FMT == QGEMV_FMT_Q6_K_R8) return (u + 31) / 32 * Q6K::TILE_BYTES;   // whole tiles
    if (FMT == QGEMV_FMT_Q4_0) return u * 36;
    return u * 68;
}

// One wave's slice of every row in the LDS-staged kernels (k_gemv_lds,
// k_gemv_dyn): units u_lo .. u_hi - 1 of a row, lane i taking units
// u_lo + i, u_lo + i + 64, ..., their activation held in registers; the
// slice's bytes sbeg .. sbeg + slen - 1 of a row move through the wave's LDS
// buffers as 16-byte chunks on a grid aligned to 16-byte global addresses
// (lane i fetches chunks i, i + 64, ...; the last one shifted back to end at
// the slice end, so no load leaves the row).  Lanes past the slice repeat its
// last unit (every load unconditional and in bounds) and drop its term.
//
// MR > 1: the lane holds the activation of MR rows (the small-M product of a
// few tokens) and dots every unit it reads from LDS against each of them.
template <int FMT, int UPL, int NL, bool NT, int MR = 1>
struct SliceStream {
    using UnitT = Unit<FMT>;
    using WT = typename UnitT::W;
    using UL = UnitLds<FMT>;
    int lane, u_lo, u_hi, sbeg, slen, nbw;
    bool empty;   // a slice past the row's last unit (see the constructor)
    ActReg<FMT> A[MR][UPL];
    int ul[UPL];
    bool ok[UPL], has1[UPL];

    __device__ __forceinline__ SliceStream(int lane_, int U, int US, int kq, int nbw_,
                                           int row_bytes)
        : lane(lane_), u_lo(kq * US), u_hi(min(U, kq * US + US)), nbw(nbw_) {
        // Slices start at tile boundaries for the repacked Q6_K, so the last
        // of WK slices can lie wholly past the row (e.g. 132 units over
        // slices of 64).  Such a slice streams the row's last tile instead
        // (whole tiles: unit_byte addresses only tile starts; its loads stay
        // inside the row and fit the slice buffers) and contributes nothing.
        empty = u_hi <= u_lo;
        if (empty) {
            constexpr int UG = FMT == QGEMV_FMT_Q6_K_R8 ? 32
                               : (FMT == QGEMV_FMT_Q4_K || FMT == QGEMV_FMT_Q6_K) ? 4 : 1;
            u_lo = (U - 1) / UG * UG;
            u_hi = U;
        }
        sbeg = unit_byte<FMT>(u_lo);
        slen = min(unit_byte<FMT>(u_hi), row_bytes) - sbeg;
    }
    // the activation of the lane's units (from global memory or LDS); MR > 1:
    // activation row m at q + m * ldq (d, s + m * ldq / 32), rows m >= mc
    // repeating row mc - 1
    __device__ __forceinline__ void load_act(const int8_t* q, const uint16_t* d,
                                             const int32_t* s, int ldq = 0, int mc = 1) {
#pragma unroll
        for (int i = 0; i < UPL; i++) {
            const int u = u_lo + lane + 64 * i;
            ok[i] = !empty && u < u_hi;
            const int uc = ok[i] ? u : u_hi - 1;
#pragma unroll
            for (int m = 0; m < MR; m++) {
                const int mm = m < mc ? m : mc - 1;
                A[m][i].load(q + (int64_t)mm * ldq, d + (int64_t)mm * (ldq / 32),
                             s + (int64_t)mm * (ldq / 32), uc);
            }
            ul[i] = uc - u_lo;
            has1[i] = 2 * uc + 1 < nbw;
        }
    }
    // offset (from the aligned chunk base) of this lane's k-th chunk
    __device__ __forceinline__ int chunk_off(int k, int delta) const {
        return min(16 * (lane + 64 * k), delta + slen - 16);
    }
    // Issue the loads of the slice of the row at rowp; returns the slice's
    // offset from the 16-byte-aligned address below it.
    __device__ __forceinline__ int stage(u32x4 (&R)[NL], const uint8_t* rowp) const {
        const uint8_t* a = rowp + sbeg;
        const int delta = (int)((uintptr_t)a & 15);
        const uint8_t* ab = a - delta;
#pragma unroll
        for (int k = 0; k < NL; k++) R[k] = ld16_stream<NT>(ab + chunk_off(k, delta));
        return delta;
    }
    // Park a staged slice in the wave's LDS buffer (in the row's byte order).
    __device__ __forceinline__ void commit(const u32x4 (&R)[NL], int delta, uint8_t* buf) const {
#pragma unroll
        for (int k = 0; k < NL; k++) st16(buf + chunk_off(k, delta), R[k]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    // The slice's dot with the activation, reduced over the wave (valid in
    // lane 63).
    __device__ __forceinline__ float dot(const uint8_t* buf, int delta) const {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < UPL; i++) {
            WT wv;
            UL::load(buf, delta, ul[i], has1[i], wv);
            const float t = UnitT::term(wv, A[0][i], u_lo + ul[i], nbw);
            acc += ok[i] ? t : 0.0f;
        }
        return group_sum<64>(acc);
    }
    // The slice's dots with the MR activation rows, each formed exactly as
    // dot() forms it for its row (valid in lane 63).
    __device__ __forceinline__ void dot_mr(const uint8_t* buf, int delta, float (&out)[MR]) const {
        float acc[MR];
#pragma unroll
        for (int m = 0; m < MR; m++) acc[m] = 0.0f;
#pragma unroll
        for (int i = 0; i < UPL; i++) {
            WT wv;
            UL::load(buf, delta, ul[i], has1[i], wv);
#pragma unroll
            for (int m = 0; m < MR; m++) {
                const float t = UnitT::term(wv, A[m][i], u_lo + ul[i], nbw);
                acc[m] += ok[i] ? t : 0.0f;
            }
        }
#pragma unroll
        for (int m = 0; m < MR; m++) out[m] = group_sum<64>(acc[m]);
    }
    // Two rows' dots (two independent chains for the scheduler to
    // interleave); each is formed exactly as dot() forms it.
    __device__ __forceinline__ void dot2(const uint8_t* buf0, int delta0, const uint8_t* buf1,
                                         int delta1, float& s0, float& s1) const {
        float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
        for (int i = 0; i < UPL; i++) {
            WT w0, w1;
            UL::load(buf0, delta0, ul[i], has1[i], w0);
            UL::load(buf1, delta1, ul[i], has1[i], w1);
            const float t0 = UnitT::term(w0, A[0][i], u_lo + ul[i], nbw);
            const float t1 = UnitT::term(w1, A[0][i], u_lo + ul[i], nbw);
            acc0 += ok[i] ? t0 : 0.0f;
            acc1 += ok[i] ? t1 : 0.0f;
        }
        s0 = group_sum<64>(acc0);
        s1 = group_sum<64>(acc1);
    }
};

// The activation quantised in the launch (XQ): the workgroup quantises x
// into LDS (aq, ad, as), every lane loads its units' activation from there,
// and workgroup 0 writes the codes out.  Called by every thread.
template <int NTH, class SS>
__device__ __forceinline__ void xq_prologue(SS& ss, const ActIn& ai, int nbw, int Kp,
                                            const f32x4 (&xv)[XqLoads<NTH>], int8_t* aq,
                                            uint16_t* ad, int32_t* as) {
    quantize_row_lds<NTH>(ai.x, 32 * nbw, Kp, xv, aq, ad, as);
    __syncthreads();
    ss.load_act(aq, ad, as);
    if (blockIdx.x == 0) xq_write_out<NTH>(ai, Kp, aq, ad, as);
}

// SwiGLU outputs of the fused gate|up product (SW).  Workgroup 0 zeroes the
// activation blocks between nh and the next multiple of 256.
template <int NTH>
__device__ __forceinline__ void swiglu_zero_tail(const SwigluOut& so) {
    const int64_t nhb = so.nh / 32, nbo = (so.nh + 255) / 256 * 8;
    for (int64_t t = threadIdx.x; t < (nbo - nhb) * 8; t += NTH) {
        const int64_t b = nhb + t / 8;
        *reinterpret_cast<uint32_t*>(so.q + 32 * b + 4 * (t % 8)) = 0u;
        if (t % 8 == 0) {
            so.d[b] = 0;
            so.s[b] = 0;
        }
    }
}

// The output blocks hb0 + j * stride (j < nblk) of the fused product: row l
// of block j (gate rows l < 32, up rows l >= 32) is parked in part at
// (64 j + l) * WK + slice, its WK slices added in slice order.  One thread per
// value forms h = silu(g) * u into hseg, then 8 lanes per block quantise it
// as the next product's activation block (the same device functions as
// k_silu_mul_quantize); [gate | up] and h are stored only where asked for.
// Called by every thread of the workgroup once part is complete.
template <int NTH, int WK>
__device__ __forceinline__ void swiglu_epilogue(const float* part, float* hseg, int nblk,
                                                int64_t hb0, int64_t stride,
                                                const SwigluOut& so) {
    for (int t = threadIdx.x; t < 32 * nblk; t += NTH) {
        const int j = t >> 5, i = t & 31;
        const int64_t hb = hb0 + j * stride;
        float g = part[(64 * j + i) * WK], u = part[(64 * j + 32 + i) * WK];
#pragma unroll
        for (int kk = 1; kk < WK; kk++) {
            g += part[(64 * j + i) * WK + kk];
            u += part[(64 * j + 32 + i) * WK + kk];
        }
        const float hv = silu_mul(g, u);
        hseg[t] = hv;
        if (so.gu) {
            so.gu[32 * hb + i] = g;
            so.gu[so.nh + 32 * hb + i] = u;
        }
        if (so.h) so.h[32 * hb + i] = hv;
    }
    __syncthreads();
    // whole aligned groups of 8 lanes take part (8 * nblk is a multiple of 8)
    for (int t = threadIdx.x; t < 8 * nblk; t += NTH) {
        const int j = t >> 3, sub = t & 7;
        const int64_t hb = hb0 + j * stride;
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; k++) v[k] = hseg[32 * j + 4 * sub + k];
        const QBlock r = quantize_block8(v);
        *reinterpret_cast<uint32_t*>(so.q + 32 * hb + 4 * sub) = r.packed;
        if (sub == 0) {
            so.d[hb] = (uint16_t)r.dbits;
            so.s[hb] = r.sum;
        }
    }
}

// LDS-streaming GEMV (whole waves per row, LPR = 64).  Same work split as
// k_gemv, but a wave brings its slice of a row in with fully coalesced loads
// -- lane i fetches the 16-byte chunk i, i + 64, ... of the slice, on a chunk
// grid aligned to 16-byte global addresses, so each wave instruction reads
// 1 KB of consecutive, aligned bytes (with the non-temporal hint, which is
// safe because whole cache lines are consumed by one instruction) -- and
// parks it in its own LDS buffer in the original byte order; the lanes then
// read their units' fields from LDS.  The last chunk is shifted back to end
// exactly at the slice end (it overlaps its neighbour; both write the same
// bytes), so no load leaves the row.  Two rows are in flight in registers
// while a third is computed from LDS.  Row results are parked in LDS and
// written out together (one lane per row would issue a store per row).
//
// SW (the fused gate|up product of a SwiGLU block): the weights are gate rows
// 0 .. nh-1 then up rows nh .. 2nh-1 (N = 2nh).  A workgroup walks whole
// output blocks of 32: block b is gate rows 32b .. 32b+31 and up rows
// nh+32b .. nh+32b+31, so the 64 row results of a block end up parked in the
// workgroup's LDS together, and at the end of a segment swiglu_epilogue turns
// them into the next product's activation blocks.
template <int FMT, int UPL, int WK, int NL, bool NT, bool SW, bool XQ>
__global__ __launch_bounds__(WG) void k_gemv_lds(const uint8_t* __restrict__ w, int N, int U,
                                                  int US, int nbw, int row_bytes, int buf_bytes,
                                                  const int8_t* __restrict__ q,
                                                  const uint16_t* __restrict__ d,
                                                  const int32_t* __restrict__ s,
                                                  float* __restrict__ y, const SwigluOut so,
                                                  const ActIn ai) {
    extern __shared__ __align__(16) uint8_t lds[];
    constexpr int LPR = 64;
    constexpr int RPP = 4 / WK;
    __shared__ float part[SEGP * RPP * WK];
    __shared__ float hseg[SW ? 32 * (SEGP * RPP / 64) : 1];   // SW: h of a segment's blocks

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kq = wave % WK, rg = wave / WK;
    SliceStream<FMT, UPL, NL, NT> ss(lane, U, US, kq, nbw, row_bytes);
    if constexpr (!XQ) ss.load_act(q, d, s);
    // XQ: the activation row, quantised in this workgroup, after the slice buffers
    const int Kp = (32 * nbw + 255) / 256 * 256;
    int8_t* const aq = reinterpret_cast<int8_t*>(lds + 8 * buf_bytes);
    uint16_t* const ad = reinterpret_cast<uint16_t*>(lds + 8 * buf_bytes + Kp);
    int32_t* const as = reinterpret_cast<int32_t*>(lds + 8 * buf_bytes + Kp + Kp / 16);

    uint8_t* buf0 = lds + (2 * wave) * buf_bytes;
    uint8_t* buf1 = buf0 + buf_bytes;
    const int64_t G = gridDim.x;
    const int64_t ngroups = ((int64_t)N + RPP - 1) / RPP;
    constexpr int GPB = 64 / RPP;   // SW: row groups (passes) per output block
    const int64_t nhb = SW ? so.nh / 32 : 0;
    const int64_t npass_all =
        SW ? (nhb > (int64_t)blockIdx.x ? (nhb - blockIdx.x + G - 1) / G : 0) * GPB
           : (ngroups > (int64_t)blockIdx.x ? (ngroups - blockIdx.x + G - 1) / G : 0);
    auto row_of = [&](int64_t p) -> int64_t {
        if (!SW) return (blockIdx.x + p * G) * RPP + rg;
        // the prefetch runs up to two passes past the last one: keep it on
        // this workgroup's last rows (cached) rather than other blocks' rows
        p = min(p, npass_all - 1);
        const int64_t hb = blockIdx.x + (p / GPB) * G;
        const int l = (int)(p % GPB) * RPP + rg;   // 0..31 gate, 32..63 up
        return l < 32 ? 32 * hb + l : so.nh + 32 * hb + (l - 32);
    };
    if (SW && blockIdx.x == 0) swiglu_zero_tail<WG>(so);
    auto stage = [&](u32x4 (&R)[NL], int64_t row) {
        return ss.stage(R, w + min(row, (int64_t)N - 1) * (int64_t)row_bytes);
    };
    auto commit = [&](const u32x4 (&R)[NL], int delta, uint8_t* buf) { ss.commit(R, delta, buf); };
    auto dot_row = [&](const uint8_t* buf, int delta) { return ss.dot(buf, delta); };
    auto finish_row = [&](float acc, int pl) {
        if (lane == LPR - 1) part[(pl * RPP + rg) * WK + kq] = acc;
    };

    static_assert(SEGP % GPB == 0, "a segment holds whole output blocks");
    for (int64_t p0 = 0; p0 < npass_all; p0 += SEGP) {
        const int np = (int)min((int64_t)SEGP, npass_all - p0);
        u32x4 Ra[NL], Rb[NL];
        int da, db, d0, d1;
        {
            // three rows requested before the first is committed (XQ: after
            // the loads of x, which is what the waves wait for first; the
            // rows stream in while the workgroup quantises x)
            const bool xq = XQ && p0 == 0;
            f32x4 xv[XqLoads<WG>];
            if (xq) xq_load(ai.x, 32 * nbw, 0, xv);
            __builtin_amdgcn_sched_barrier(0);
            u32x4 Rc[NL];
            const int dc = stage(Rc, row_of(p0));
            __builtin_amdgcn_sched_barrier(0);
            da = stage(Ra, row_of(p0 + 1));
            __builtin_amdgcn_sched_barrier(0);
            db = stage(Rb, row_of(p0 + 2));
            __builtin_amdgcn_sched_barrier(0);
            if (xq) xq_prologue<WG>(ss, ai, nbw, Kp, xv, aq, ad, as);
            commit(Rc, dc, buf0);
            d0 = dc;
        }
        for (int p = 0; p < np; p += 2) {
            finish_row(dot_row(buf0, d0), p);
            commit(Ra, da, buf1);
            d1 = da;
            da = stage(Ra, row_of(p0 + p + 3));
            __builtin_amdgcn_sched_barrier(0);
            if (p + 1 < np) finish_row(dot_row(buf1, d1), p + 1);
            commit(Rb, db, buf0);
            d0 = db;
            db = stage(Rb, row_of(p0 + p + 4));
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        if (!SW) {
            for (int t = threadIdx.x; t < np * RPP; t += WG) {
                const int64_t row = (blockIdx.x + (p0 + t / RPP) * G) * RPP + t % RPP;
                if (row < N) {
                    float v = part[t * WK];
#pragma unroll
                    for (int k = 1; k < WK; k++) v += part[t * WK + k];
                    y[row] = v;
                }
            }
        } else {
            // row l of the segment's output block j is part[(64 j + l) * WK + kq]
            swiglu_epilogue<WG, WK>(part, hseg, np / GPB, blockIdx.x + (p0 / GPB) * G, G, so);
        }
        __syncthreads();
    }
}

// Dynamic-row LDS-streaming GEMV: one workgroup of DW = 8 waves per compute
// unit, the same per-row work as k_gemv_lds, but the rows of a workgroup are
// handed to its waves from a counter in LDS, one at a time or (PAIRS, short
// slices) two consecutive ones, whose dots are computed together.  With two
// 4-wave workgroups per compute unit and a fixed share each, the workgroup
// dispatched first ran 16-36% faster than its co-resident twin (its waves
// are older and win the issue arbitration), and the unit finished with the
// slow one; pulling rows from a shared counter lets every wave of the unit
// work until the unit's rows are done.  A workgroup owns the row groups of
// DRG rows b, b + G, b + 2G, ...; with split-K (WK > 1) each of the WK
// slices of a row has its own counter (the waves holding that slice's
// activation pull from it) and the slices' partial sums meet in LDS, added
// in slice order as in k_gemv_lds, so every output has the same bits.
//
// SW (the fused gate|up product, as in k_gemv_lds): a workgroup owns the
// output blocks b, b + G, b + 2G, ... (64 rows each, gate then up); every row
// result goes to LDS and swiglu_epilogue forms and quantises h once all of
// them are in.  With two 4-wave workgroups per unit and whole blocks each,
// the younger workgroup of a unit ran ~4 us behind its twin (and 448 blocks
// do not split evenly over 512 workgroups); here the unit's 8 waves share
// its one or two blocks until the last row.
constexpr int DW = 8;           // waves of a dynamic-row workgroup
constexpr int DWG = 64 * DW;    // its threads
constexpr int DRG = 8;          // rows per row group of the static split
static_assert(DRG % 2 == 0, "pairs of rows stay inside a row group");

//
// MR > 1 (the small-M product of MR activation rows, row m at q + m * ldq,
// output row m at y + m * N; rows m >= mc are computed on row mc - 1 and not
// stored): every unit read from LDS is dotted against the MR rows, each dot
// formed exactly as the batch-1 product forms it, so output row m has the
// bits of the batch-1 product on activation row m with the same slices.
template <int FMT, int UPL, int WK, int NL, bool XQ, bool SW, bool PAIRS, int MR = 1>
__global__ __launch_bounds__(DWG) void k_gemv_dyn(const uint8_t* __restrict__ w, int N, int U,
                                                   int US, int nbw, int row_bytes, int buf_bytes,
                                                   const int8_t* __restrict__ q,
                                                   const uint16_t* __restrict__ d,
                                                   const int32_t* __restrict__ s,
                                                   float* __restrict__ y, const SwigluOut so,
                                                   const ActIn ai, int ldq, int mc) {
    static_assert(DW % WK == 0, "whole waves per slice");
    static_assert(MR == 1 || (!XQ && !SW && !PAIRS), "several activation rows: plain rows");
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ int cnt[WK];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kq = wave % WK;
    SliceStream<FMT, UPL, NL, true, MR> ss(lane, U, US, kq, nbw, row_bytes);

    // this workgroup's rows; indices past them (and rows past N) map to row
    // N - 1, whose bytes the prefetch then reads from cache
    const int G = gridDim.x, b = blockIdx.x;
    const int nhb = SW ? (int)(so.nh / 32) : 0;
    const int nblk = SW ? (nhb > b ? (nhb - b + G - 1) / G : 0) : 0;   // SW: output blocks
    const int ngr = (N + DRG - 1) / DRG;
    const int pool_n = SW ? 64 * nblk : (ngr > b ? (ngr - b + G - 1) / G * DRG : 0);
    auto row_raw = [&](int i) {
        if constexpr (SW) {
            const int hb = b + (i >> 6) * G, l = i & 63;
            return l < 32 ? 32 * hb + l : (int)so.nh + 32 * hb + (l - 32);
        }
        return DRG * (b + (i / DRG) * G) + i % DRG;
    };
    auto row_of = [&](int i) { return i < pool_n ? min(row_raw(i), N - 1) : N - 1; };

    if (threadIdx.x < WK) cnt[threadIdx.x] = 0;
    if (SW && b == 0) swiglu_zero_tail<DWG>(so);
    if constexpr (!XQ) ss.load_act(q, d, s, ldq, mc);
    const int Kp = (32 * nbw + 255) / 256 * 256;
    int8_t* const aq = reinterpret_cast<int8_t*>(lds + 2 * DW * buf_bytes);
    uint16_t* const ad = reinterpret_cast<uint16_t*>(lds + 2 * DW * buf_bytes + Kp);
    int32_t* const as = reinterpret_cast<int32_t*>(lds + 2 * DW * buf_bytes + Kp + Kp / 16);
    float* const part =
        reinterpret_cast<float*>(lds + 2 * DW * buf_bytes + (XQ ? act_lds_bytes(Kp) : 0));
    float* const hseg = part + pool_n * WK;   // SW: h of the workgroup's blocks
    uint8_t* buf0 = lds + (2 * wave) * buf_bytes;
    uint8_t* buf1 = buf0 + buf_bytes;
    __syncthreads();   // the counters are zero

    // the next row index of this wave's slice: one LDS atomic per row,
    // issued a step before its value is read (take) so that its latency
    // stays off the path to the row's loads
    auto grab_issue = [&]() {
        int v = 0;
        if (lane == 0) v = atomicAdd(&cnt[kq], 1);
        return v;
    };
    auto take = [&](int v) { return __builtin_amdgcn_readfirstlane(v); };
    auto grab = [&]() { return take(grab_issue()); };
    auto stage = [&](u32x4 (&R)[NL], int row) {
        return ss.stage(R, w + (int64_t)row * row_bytes);
    };
    auto commit = [&](const u32x4 (&R)[NL], int delta, uint8_t* buf) { ss.commit(R, delta, buf); };
    auto dot_row = [&](const uint8_t* buf, int delta) { return ss.dot(buf, delta); };
    auto finish_row = [&](float acc, int i) {
        if (lane == 63 && i < pool_n && row_raw(i) < N) {
            if constexpr (WK == 1 && !SW) y[row_raw(i)] = acc;
            else part[i * WK + kq] = acc;
        }
    };
    // a row's dot(s) with the activation row(s), stored or parked
    auto row_done = [&](const uint8_t* buf, int delta, int i) {
        if constexpr (MR == 1) {
            finish_row(dot_row(buf, delta), i);
        } else {
            float v[MR];
            ss.dot_mr(buf, delta, v);
            if (lane == 63 && i < pool_n && row_raw(i) < N) {
#pragma unroll
                for (int m = 0; m < MR; m++) {
                    if (m < mc) {
                        if constexpr (WK == 1) y[(int64_t)m * N + row_raw(i)] = v[m];
                        else part[(i * WK + kq) * MR + m] = v[m];
                    }
                }
            }
        }
    };

    if constexpr (PAIRS) {
        // rows go in pairs of consecutive indices (one LDS atomic per pair;
        // pools and their row groups have even sizes, so a pair never
        // straddles the end of the pool); two pairs are in flight while a
        // third is computed, its two dots interleaved
        auto grab2_issue = [&]() {
            int v = 0;
            if (lane == 0) v = atomicAdd(&cnt[kq], 2);
            return v;
        };
        u32x4 A0[NL], B0[NL], A1[NL], B1[NL];
        int j0, j1, dA0, dB0, dA1, dB1;
        {
            // four rows requested before the first is committed (XQ: after
            // the loads of x; the rows stream in while x is quantised)
            f32x4 xv[XqLoads<DWG>];
            if (XQ) xq_load<DWG>(ai.x, 32 * nbw, 0, xv);
            __builtin_amdgcn_sched_barrier(0);
            j0 = take(grab2_issue());
            dA0 = stage(A0, row_of(j0));
            dB0 = stage(B0, row_of(j0 + 1));
            __builtin_amdgcn_sched_barrier(0);
            j1 = take(grab2_issue());
            dA1 = stage(A1, row_of(j1));
            dB1 = stage(B1, row_of(j1 + 1));
            __builtin_amdgcn_sched_barrier(0);
            if (XQ) xq_prologue<DWG>(ss, ai, nbw, Kp, xv, aq, ad, as);
        }
        int tn = grab2_issue();   // the pair after j1, in flight
        // A wave's indices increase (j0 < j1 at the loop head), so once one is
        // past the pool all later are.  The loop runs while both pairs in
        // flight are rows of the pool and has no other exit: with an exit
        // between its halves the two ways out met the back edge in one block,
        // with the register sets in opposite load order, and the compiler's
        // wait counts drained every load at the loop head (one pair in flight
        // instead of two).  The last pair, if any, is finished after it.
        while (j1 < pool_n) {
            commit(A0, dA0, buf0);
            commit(B0, dB0, buf1);
            const int c0 = j0, e0 = dA0, f0 = dB0;
            j0 = take(tn);
            tn = grab2_issue();
            dA0 = stage(A0, row_of(j0));
            dB0 = stage(B0, row_of(j0 + 1));
            __builtin_amdgcn_sched_barrier(0);
            {
                float s0, s1;
                ss.dot2(buf0, e0, buf1, f0, s0, s1);
                finish_row(s0, c0);
                finish_row(s1, c0 + 1);
            }
            commit(A1, dA1, buf0);
            commit(B1, dB1, buf1);
            const int c1 = j1, e1 = dA1, f1 = dB1;
            j1 = take(tn);
            tn = grab2_issue();
            dA1 = stage(A1, row_of(j1));
            dB1 = stage(B1, row_of(j1 + 1));
            __builtin_amdgcn_sched_barrier(0);
            {
                float s0, s1;
                ss.dot2(buf0, e1, buf1, f1, s0, s1);
                finish_row(s0, c1);
                finish_row(s1, c1 + 1);
            }
        }
        if (j0 < pool_n) {
            commit(A0, dA0, buf0);
            commit(B0, dB0, buf1);
            float s0, s1;
            ss.dot2(buf0, dA0, buf1, dB0, s0, s1);
            finish_row(s0, j0);
            finish_row(s1, j0 + 1);
        }
    } else {
        u32x4 Ra[NL], Rb[NL];
        int ia, ib, i0, d0, d1, da, db;
        {
            // three rows requested before the first is committed (XQ: after the
            // loads of x; the rows stream in while the workgroup quantises x)
            f32x4 xv[XqLoads<DWG>];
            if (XQ) xq_load<DWG>(ai.x, 32 * nbw, 0, xv);
            __builtin_amdgcn_sched_barrier(0);
            u32x4 Rc[NL];
            const int ic = grab();
            const int dc = stage(Rc, row_of(ic));
            __builtin_amdgcn_sched_barrier(0);
            ia = grab();
            da = stage(Ra, row_of(ia));
            __builtin_amdgcn_sched_barrier(0);
            ib = grab();
            db = stage(Rb, row_of(ib));
            __builtin_amdgcn_sched_barrier(0);
            if (XQ) xq_prologue<DWG>(ss, ai, nbw, Kp, xv, aq, ad, as);
            commit(Rc, dc, buf0);
            d0 = dc;
            i0 = ic;
        }
        int tn = grab_issue();   // the index after ib, in flight
        // a wave's indices increase, so once one is past the pool all later are
        while (i0 < pool_n) {
            row_done(buf0, d0, i0);
            commit(Ra, da, buf1);
            d1 = da;
            const int i1 = ia;
            ia = take(tn);
            tn = grab_issue();
            da = stage(Ra, row_of(ia));
            __builtin_amdgcn_sched_barrier(0);
            if (i1 < pool_n) row_done(buf1, d1, i1);
            commit(Rb, db, buf0);
            d0 = db;
            i0 = ib;
            ib = take(tn);
            tn = grab_issue();
            db = stage(Rb, row_of(ib));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if constexpr (SW) {
        __syncthreads();
        swiglu_epilogue<DWG, WK>(part, hseg, nblk, b, G, so);
    } else if constexpr (WK > 1) {
        __syncthreads();
        for (int t = threadIdx.x; t < pool_n * MR; t += DWG) {
            const int i = t / MR, m = t % MR;
            if (row_raw(i) < N && m < mc) {
                float v = part[i * WK * MR + m];
#pragma unroll
                for (int k = 1; k < WK; k++) v += part[(i * WK + k) * MR + m];
                y[(int64_t)m * N + row_raw(i)] = v;
            }
        }
    }
}

// ------------------------------------------------------------- launchers --

static int row_bytes_of(int fmt, int64_t K) {
    const int64_t Kp = (K + 255) / 256 * 256;
    switch (fmt) {
    case QGEMV_FMT_Q4_0: return (int)(K / 32 * 18);
    case QGEMV_FMT_Q8_0: return (int)(K / 32 * 34);
    case QGEMV_FMT_Q4_K: return (int)(Kp / 256 * 144);
    case QGEMV_FMT_Q6_K_R8: return (int)((Kp / 256 + 7) / 8 * Q6K::TILE_BYTES);
    default: return (int)(Kp / 256 * 210);
    }
}

static int units_of(int fmt, int64_t K) {
    const int64_t Kp = (K + 255) / 256 * 256;
    if (fmt == QGEMV_FMT_Q4_K || fmt == QGEMV_FMT_Q6_K || fmt == QGEMV_FMT_Q6_K_R8)
        return (int)(Kp / 64);
    return (int)((K + 63) / 64);
}

// Workgroups of one kernel instantiation that fit on the device at once
// (occupancy x compute units), cached per device.
// Units per split-K slice, the same in every kernel so that a row's slice
// sums, and so its bits, do not depend on the kernel: slices of the K-quant
// formats start at super-block boundaries, those of the repacked Q6_K at
// tile boundaries.
template <int FMT>
static int slice_units(int U, int WK) {
    int us = (U + WK - 1) / WK;
    if (FMT == QGEMV_FMT_Q4_K || FMT == QGEMV_FMT_Q6_K) us = (us + 3) / 4 * 4;
    if (FMT == QGEMV_FMT_Q6_K_R8) us = (us + 31) / 32 * 32;
    return us;
}

template <int FMT, int LPR, int UPL, int WK, bool XQ = false, bool MULTI = false>
static int resident_workgroups() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1024;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, k_gemv<FMT, LPR, UPL, WK, XQ, MULTI>, WG, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        per_cu <= 0 || cus <= 0) {
        (void)hipGetLastError();
        return 1024;
    }
    v = per_cu * cus;
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

template <int FMT, int LPR, int UPL, int WK, bool XQ = false, bool MULTI = false>
static hipError_t launch_gemv_cfg(const GemvArgs& a, int U, hipStream_t st,
                                  const ActIn& ai = ActIn{}, const MultiRows& mr = MultiRows{}) {
    constexpr int RPP = (4 / WK) * (64 / LPR);
    const int64_t ngroups = (a.N + RPP - 1) / RPP;
    // as many workgroups as fit at once, then evened out so that every
    // workgroup gets the same number of passes (to within one)
    const int64_t resident = resident_workgroups<FMT, LPR, UPL, WK, XQ, MULTI>();
    const int64_t passes = (ngroups + resident - 1) / resident;
    const int64_t grid = (ngroups + passes - 1) / passes;
    launch_kernel((k_gemv<FMT, LPR, UPL, WK, XQ, MULTI>), dim3((unsigned)grid), dim3(WG), 0,
                  st, (const uint8_t*)a.w, (int)a.N, U, slice_units<FMT>(U, WK),
                  (int)(a.K / 32), row_bytes_of(FMT, a.K), a.q, a.d, a.s, a.y, ai, mr);
    return hipGetLastError();
}

// Selection of the LDS-streaming kernels (rows of at least 33 units) and of
// their non-temporal weight loads.
constexpr bool kLdsStream = true;
constexpr bool kStreamNT = true;

// Occupancy of an LDS-streaming instantiation depends on its dynamic LDS,
// which varies with K inside one instantiation, so the cache is keyed by
// (device, LDS bytes).
template <int FMT, int UPL, int WK, int NL, bool SW, bool XQ>
static int resident_workgroups_lds(int smem) {
    static std::mutex mu;
    static std::map<std::pair<int, int>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 1024;
    }
    {
        std::lock_guard<std::mutex> lk(mu);
        const auto it = cache.find({dev, smem});
        if (it != cache.end()) return it->second;
    }
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, k_gemv_lds<FMT, UPL, WK, NL, kStreamNT, SW, XQ>, WG, smem) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        per_cu <= 0 || cus <= 0) {
        (void)hipGetLastError();
        return 1024;
    }
    const int v = per_cu * cus;
    std::lock_guard<std::mutex> lk(mu);
    cache[{dev, smem}] = v;
    return v;
}

// Workgroups per compute unit for the LDS-streaming kernels.  Measured on
// MI355X: two workgroups (8 waves) per CU stream the Llama-shaped matrices
// fastest; more waves add in-flight requests without adding bandwidth.
constexpr int kLdsWgPerCu = 2;

template <int FMT, int UPL, int WK, int NL, bool SW, bool XQ>
static hipError_t launch_lds_cfg(const GemvArgs& a, const SwigluOut& so, const ActIn& ai, int U,
                                 int US, int buf_bytes, hipStream_t st) {
    constexpr int RPP = 4 / WK;
    const int Kp = (int)((a.K + 255) / 256 * 256);
    // 4 waves x 2 slice buffers, then (XQ) the quantised activation row
    const int smem = 8 * buf_bytes + (XQ ? act_lds_bytes(Kp) : 0);
    // work items: row groups, or (SW) output blocks of 32
    const int64_t items = SW ? so.nh / 32 : (a.N + RPP - 1) / RPP;
    int64_t resident = resident_workgroups_lds<FMT, UPL, WK, NL, SW, XQ>(smem);
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        cus > 0 && resident > (int64_t)kLdsWgPerCu * cus)
        resident = (int64_t)kLdsWgPerCu * cus;
    const int64_t passes = (items + resident - 1) / resident;
    const int64_t grid = (items + passes - 1) / passes;
    launch_kernel((k_gemv_lds<FMT, UPL, WK, NL, kStreamNT, SW, XQ>), dim3((unsigned)grid),
                  dim3(WG), smem, st, (const uint8_t*)a.w, (int)a.N, U, US, (int)(a.K / 32),
                  row_bytes_of(FMT, a.K), buf_bytes, a.q, a.d, a.s, a.y, so, ai);
    return hipGetLastError();
}

// Host view of the row slices of the LDS-streaming kernel.
struct SliceGeom {
    int US;       // units per slice
    int nchunk;   // most 16-byte chunks a slice (plus its misalignment) spans
};

template <int FMT>
static SliceGeom slice_geom(int64_t K, int U, int WK) {
    const int rb = row_bytes_of(FMT, K);
    SliceGeom g;
    g.US = slice_units<FMT>(U, WK);
    g.nchunk = 0;
    for (int k = 0; k < WK; k++) {
        const int lo = k * g.US;
        if (lo >= U) break;
        const int hi = lo + g.US < U ? lo + g.US : U;
        int e = unit_byte<FMT>(hi);
        if (e > rb) e = rb;
        const int len = e - unit_byte<FMT>(lo);
        const int nc = (len + 15 + 15) / 16;  // up to 15 bytes of misalignment
        if (nc > g.nchunk) g.nchunk = nc;
    }
    return g;
}

// The LDS-streaming kernels take at most 8 chunks per lane and 8 slice
// buffers (each with 16 bytes of slack for the aligned-dword field reads),
// plus the quantised activation row when they form it themselves, within
// 64 KB of LDS minus the parked row results.
template <int FMT>
static bool lds_slice_fits(const SliceGeom& g, int act_bytes = 0) {
    return (g.nchunk + 63) / 64 <= 8 && 8 * (16 * g.nchunk + 16) + act_bytes <= 65536 - 8192;
}

template <int FMT, int UPL, int WK, bool SW = false, bool XQ = false>
static hipError_t launch_lds_wk(const GemvArgs& a, int U, const SliceGeom& g, hipStream_t st,
                                const SwigluOut& so = SwigluOut{}, const ActIn& ai = ActIn{}) {
    const int buf_bytes = 16 * g.nchunk + 16;
    const int nl = (g.nchunk + 63) / 64;  // 16-byte chunks per lane
    if (nl <= 2) return launch_lds_cfg<FMT, UPL, WK, 2, SW, XQ>(a, so, ai, U, g.US, buf_bytes, st);
    if (nl <= 3) return launch_lds_cfg<FMT, UPL, WK, 3, SW, XQ>(a, so, ai, U, g.US, buf_bytes, st);
    if (nl <= 4) return launch_lds_cfg<FMT, UPL, WK, 4, SW, XQ>(a, so, ai, U, g.US, buf_bytes, st);
    if (nl <= 6) return launch_lds_cfg<FMT, UPL, WK, 6, SW, XQ>(a, so, ai, U, g.US, buf_bytes, st);
    return launch_lds_cfg<FMT, UPL, WK, 8, SW, XQ>(a, so, ai, U, g.US, buf_bytes, st);
}

// Split-K of the LDS-streaming kernel: waves per row, by the row's length in
// 64-weight units of 36 bytes (a Q8_0 unit, 68 bytes, counts twice: 14336 x
// 4096 ran 12.6 against 13.1 us with two waves per row).
template <int FMT>
static int wk_units(int U) { return FMT == QGEMV_FMT_Q8_0 ? 2 * U : U; }
template <int FMT>
static int lds_wk(int U) {
    const int Uw = wk_units<FMT>(U);
    return Uw > 128 ? 4 : (Uw > 64 ? 2 : 1);
}

// Compute units of the current device (cached per device).
static int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0) {
        (void)hipGetLastError();
        return 256;
    }
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

// The dynamic-row kernel: one workgroup per compute unit.  Returns
// hipErrorNotSupported (nothing launched) where its slice buffers, the
// activation row and the partial sums would not fit in 64 KB of LDS.
// Slices of at most this many bytes go through the dynamic-row kernel two
// rows at a time per wave (four rows in flight instead of two).  Measured on
// MI355X: the 2304-byte rows of the fused gate|up product ran ~1 us faster
// in pairs; the 3360-byte rows of the lm_head ran ~2.5 us slower (eight waves
// with two of its rows in flight each already keep ~54 KB per unit in
// flight).
constexpr int kDynPairMaxSlice = 3072;

template <int FMT, int UPL, int WK, int NL, bool XQ, bool SW>
static hipError_t launch_dyn_cfg(const GemvArgs& a, const SwigluOut& so, const ActIn& ai, int U,
                                 int US, int buf_bytes, hipStream_t st) {
    const int cus = cu_count();
    // work items: row groups of DRG, or (SW) output blocks of 64 rows
    const int64_t items = SW ? so.nh / 32 : (a.N + DRG - 1) / DRG;
    const int64_t grid = items < cus ? items : cus;
    const int64_t per_wg = (items + grid - 1) / grid;
    const int64_t pool_cap = per_wg * (SW ? 64 : DRG);
    const int Kp = (int)((a.K + 255) / 256 * 256);
    const int64_t smem = 2 * DW * (int64_t)buf_bytes + (XQ ? act_lds_bytes(Kp) : 0) +
                         (WK > 1 || SW ? pool_cap * WK * 4 : 0) + (SW ? per_wg * 32 * 4 : 0);
    if (smem > 65536 - 64) return hipErrorNotSupported;
    if (buf_bytes - 32 <= kDynPairMaxSlice)
        launch_kernel((k_gemv_dyn<FMT, UPL, WK, NL, XQ, SW, true>), dim3((unsigned)grid),
                      dim3(DWG), (unsigned)smem, st, (const uint8_t*)a.w, (int)a.N, U, US,
                      (int)(a.K / 32), row_bytes_of(FMT, a.K), buf_bytes, a.q, a.d, a.s, a.y,
                      so, ai, 0, 1);
    else
        launch_kernel((k_gemv_dyn<FMT, UPL, WK, NL, XQ, SW, false>), dim3((unsigned)grid),
                      dim3(DWG), (unsigned)smem, st, (const uint8_t*)a.w, (int)a.N, U, US,
                      (int)(a.K / 32), row_bytes_of(FMT, a.K), buf_bytes, a.q, a.d, a.s, a.y,
                      so, ai, 0, 1);
    return hipGetLastError();
}

template <int FMT, int UPL, int WK, bool XQ, bool SW>
static hipError_t launch_dyn_wk(const GemvArgs& a, int U, const SliceGeom& g, hipStream_t st,
                                const SwigluOut& so, const ActIn& ai) {
    const int buf_bytes = 16 * g.nchunk + 16;
    const int nl = (g.nchunk + 63) / 64;
    if (nl <= 2) return launch_dyn_cfg<FMT, UPL, WK, 2, XQ, SW>(a, so, ai, U, g.US, buf_bytes, st);
    if (nl <= 3) return launch_dyn_cfg<FMT, UPL, WK, 3, XQ, SW>(a, so, ai, U, g.US, buf_bytes, st);
    if (nl <= 4) return launch_dyn_cfg<FMT, UPL, WK, 4, XQ, SW>(a, so, ai, U, g.US, buf_bytes, st);
    return hipErrorNotSupported;
}

// Matrices with at least this many rows per compute unit take the
// dynamic-row kernel (where it fits).  Measured on MI355X: it ends the
// 128256-row lm_head 2-3 us sooner (62.4 vs 64.8 us), but runs the
// 28672 x 4096 gate|up product 1.2-1.4 us slower than two 4-wave workgroups
// per unit with fixed shares, and the 4096-row down product no faster.
constexpr int kDynRowsPerCu = 256;

template <int FMT, bool SW, bool XQ>
static hipError_t launch_lds_fmt(const GemvArgs& a, int U, const SliceGeom& g, hipStream_t st,
                                 const SwigluOut& so, const ActIn& ai) {
    // the fused gate|up product always tries the dynamic-row kernel (whole
    // output blocks per unit, shared by its 8 waves)
    // (the split-K matches lds_wk: g was formed with it)
    const int Uw = wk_units<FMT>(U);
    if (SW || a.N >= (int64_t)kDynRowsPerCu * cu_count()) {
        hipError_t e = hipErrorNotSupported;
        if (U > 256) e = launch_dyn_wk<FMT, 2, 4, XQ, SW>(a, U, g, st, so, ai);
        else if (Uw > 128) e = launch_dyn_wk<FMT, 1, 4, XQ, SW>(a, U, g, st, so, ai);
        else if (Uw > 64) e = launch_dyn_wk<FMT, 1, 2, XQ, SW>(a, U, g, st, so, ai);
        else e = launch_dyn_wk<FMT, 1, 1, XQ, SW>(a, U, g, st, so, ai);
        if (e != hipErrorNotSupported) return e;
    }
    if (U > 256) return launch_lds_wk<FMT, 2, 4, SW, XQ>(a, U, g, st, so, ai);
    if (Uw > 128) return launch_lds_wk<FMT, 1, 4, SW, XQ>(a, U, g, st, so, ai);
    if (Uw > 64) return launch_lds_wk<FMT, 1, 2, SW, XQ>(a, U, g, st, so, ai);
    return launch_lds_wk<FMT, 1, 1, SW, XQ>(a, U, g, st, so, ai);
}

// Repacked Q6_K rows of 129 to 256 units (split-K over 4 waves) that are too
// few to take the dynamic-row kernel go through the direct-load kernel: the
// repacked fields load per lane as aligned 16-byte pieces, and as many
// workgroups as fit keep the units busy.  Measured on MI355X (the 4096 x
// 14336 down product in the decode step, same GPU and process): 11.2-11.3 us against
// 11.8-11.9 us through LDS (same slices, same bits); with a third row buffer
// (two rows in flight) 12.7 us.
constexpr bool kDirectR8Long = true;

template <int FMT>
static hipError_t launch_gemv_fmt(const GemvArgs& a, hipStream_t st) {
    const int U = units_of(FMT, a.K);
    if (FMT == QGEMV_FMT_Q6_K_R8 && kDirectR8Long && U > 128 && U <= 256 &&
        a.N < (int64_t)kDynRowsPerCu * cu_count())
        return launch_gemv_cfg<FMT, 64, 1, 4>(a, U, st);
    if (kLdsStream && U > 32) {
        const SliceGeom g = slice_geom<FMT>(a.K, U, lds_wk<FMT>(U));
        if (lds_slice_fits<FMT>(g)) return launch_lds_fmt<FMT, false, false>(a, U, g, st, {}, {});
    }
    if (U > 256) return launch_gemv_cfg<FMT, 64, 2, 4>(a, U, st);
    if (U > 128) return launch_gemv_cfg<FMT, 64, 1, 4>(a, U, st);
    if (U > 64) return launch_gemv_cfg<FMT, 64, 1, 2>(a, U, st);
    if (U > 32) return launch_gemv_cfg<FMT, 64, 1, 1>(a, U, st);
    if (U > 16) return launch_gemv_cfg<FMT, 32, 1, 1>(a, U, st);
    if (U > 8) return launch_gemv_cfg<FMT, 16, 1, 1>(a, U, st);
    if (U > 4) return launch_gemv_cfg<FMT, 8, 1, 1>(a, U, st);
    return launch_gemv_cfg<FMT, 4, 1, 1>(a, U, st);
}

// Quantise x and multiply in one launch where the rows take the LDS-streaming
// kernel and its LDS also holds the activation row; otherwise the two
// launches it stands for (same bits either way).
template <int FMT>
static hipError_t launch_quantize_gemv_fmt(const GemvArgs& a, const ActIn& ai, hipStream_t st) {
    const int U = units_of(FMT, a.K);
    const int Kp = (int)((a.K + 255) / 256 * 256);
    if (kLdsStream && U > 32) {
        const SliceGeom g = slice_geom<FMT>(a.K, U, lds_wk<FMT>(U));
        if (lds_slice_fits<FMT>(g, act_lds_bytes(Kp)))
            return launch_lds_fmt<FMT, false, true>(a, U, g, st, {}, ai);
    } else if (U <= 32 && Kp <= kXqShortKp) {
        // short rows: the lanes-per-row kernel, same mapping as the GEMV
        if (U > 16) return launch_gemv_cfg<FMT, 32, 1, 1, true>(a, U, st, ai);
        if (U > 8) return launch_gemv_cfg<FMT, 16, 1, 1, true>(a, U, st, ai);
        if (U > 4) return launch_gemv_cfg<FMT, 8, 1, 1, true>(a, U, st, ai);
        return launch_gemv_cfg<FMT, 4, 1, 1, true>(a, U, st, ai);
    }
    hipError_t e = launch_quantize_act(ai.x, 1, a.K, a.K, ai.q, ai.d, ai.s, st);
    if (e != hipSuccess) return e;
    GemvArgs b = a;
    b.q = ai.q;
    b.d = ai.d;
    b.s = ai.s;
    return launch_gemv_fmt<FMT>(b, st);
}

// Several matrices sharing one activation row: one launch of the
// lanes-per-row kernel over their combined rows (rows of at most 32 units),
// else one launch per matrix.
template <int FMT, bool XQ>
static hipError_t launch_multi_fmt(const MultiRows& mr, int64_t K, const int8_t* q,
                                   const uint16_t* d, const int32_t* s, const ActIn& ai,
                                   hipStream_t st) {
    const int U = units_of(FMT, K);
    const int Kp = (int)((K + 255) / 256 * 256);
    const int64_t total = mr.start[mr.count];
    if (U <= 32 && (!XQ || Kp <= kXqShortKp)) {
        const GemvArgs a{nullptr, total, K, q, d, s, nullptr};
        if (U > 16) return launch_gemv_cfg<FMT, 32, 1, 1, XQ, true>(a, U, st, ai, mr);
        if (U > 8) return launch_gemv_cfg<FMT, 16, 1, 1, XQ, true>(a, U, st, ai, mr);
        if (U > 4) return launch_gemv_cfg<FMT, 8, 1, 1, XQ, true>(a, U, st, ai, mr);
        return launch_gemv_cfg<FMT, 4, 1, 1, XQ, true>(a, U, st, ai, mr);
    }
    // one launch per matrix; with XQ the first matrix that has rows
    // quantises x and writes the codes, which the later ones read (an empty
    // matrix launches nothing, so it cannot be the one)
    bool quantised = false;
    for (int i = 0; i < mr.count; i++) {
        const int64_t n = mr.start[i + 1] - mr.start[i];
        if (n == 0) continue;
        hipError_t e;
        if (XQ && !quantised) {
            const GemvArgs a{mr.w[i], n, K, ai.q, ai.d, ai.s, mr.y[i]};
            e = launch_quantize_gemv(FMT, a, ai, st);
            quantised = true;
        } else {
            const GemvArgs a{mr.w[i], n, K, XQ ? ai.q : q, XQ ? ai.d : d, XQ ? ai.s : s, mr.y[i]};
            e = launch_gemv(FMT, a, st);
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}


// The per-format launchers one translation unit instantiates.
#define QGEMV_GEMV_FORMAT_ENTRIES(NAME, FMT)                                                  \
    hipError_t launch_gemv_##NAME(const GemvArgs& a, hipStream_t st) {                        \
        return launch_gemv_fmt<FMT>(a, st);                                                   \
    }                                                                                         \
    hipError_t launch_quantize_gemv_##NAME(const GemvArgs& a, const ActIn& ai,                \
                                           hipStream_t st) {                                  \
        return launch_quantize_gemv_fmt<FMT>(a, ai, st);                                      \
    }                                                                                         \
    hipError_t launch_multi_##NAME(const MultiRows& mr, int64_t K, const int8_t* q,           \
                                   const uint16_t* d, const int32_t* s, hipStream_t st) {     \
        return launch_multi_fmt<FMT, false>(mr, K, q, d, s, {}, st);                          \
    }                                                                                         \
    hipError_t launch_quantize_multi_##NAME(const MultiRows& mr, int64_t K, const ActIn& ai,  \
                                            hipStream_t st) {                                 \
        return launch_multi_fmt<FMT, true>(mr, K, nullptr, nullptr, nullptr, ai, st);         \
    }

#define QGEMV_GEMV_FORMAT_DECLS(NAME)                                                         \
    hipError_t launch_gemv_##NAME(const GemvArgs& a, hipStream_t st);                         \
    hipError_t launch_quantize_gemv_##NAME(const GemvArgs& a, const ActIn& ai, hipStream_t st); \
    hipError_t launch_multi_##NAME(const MultiRows& mr, int64_t K, const int8_t* q,           \
                                   const uint16_t* d, const int32_t* s, hipStream_t st);      \
    hipError_t launch_quantize_multi_##NAME(const MultiRows& mr, int64_t K, const ActIn& ai,  \
                                            hipStream_t st);
QGEMV_GEMV_FORMAT_DECLS(q4_0)
QGEMV_GEMV_FORMAT_DECLS(q4_k)
QGEMV_GEMV_FORMAT_DECLS(q6_k)
QGEMV_GEMV_FORMAT_DECLS(q6_k_r8)
QGEMV_GEMV_FORMAT_DECLS(q8_0)

}  // namespace qgemv
