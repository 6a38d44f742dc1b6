// k_small_m_rows.hip -- the DOT4 variant of the small-M product: a few
// activation rows through the dynamic-row streaming kernel of the batch-1
// GEMV (k_gemv.h), each weight row read from HBM once per group of up to
// four activation rows and each of its units dotted against all of them
// with v_dot4 ("Backends and hardware", section "CUDA": the W4A8 inner
// product on 4 x int8 dots; colibri GPU backends, eligibility gates: output
// row m is the batch-1 product on activation row m).
#include "k_gemv.h"

namespace qgemv {

namespace {

// The chunks per lane of the slice buffers: enough for every slice of at
// most 64 units (a shorter slice repeats its last chunk).
template <int FMT>
constexpr int rows_nl() {
    return FMT == QGEMV_FMT_Q6_K ? 4 : 3;
}

template <int FMT, int WK, int MR>
hipError_t launch_rows_cfg(const void* w, int64_t N, int64_t K, int64_t M, const int8_t* q,
                           const uint16_t* d, const int32_t* s, float* y, hipStream_t st) {
    constexpr int NL = rows_nl<FMT>();
    const int U = units_of(FMT, K);
    const SliceGeom g = slice_geom<FMT>(K, U, WK);
    if ((g.nchunk + 63) / 64 > NL) return hipErrorNotSupported;
    const int buf_bytes = 16 * g.nchunk + 16;
    const int cus = cu_count();
    const int64_t items = (N + DRG - 1) / DRG;
    const int64_t grid = items < cus ? items : cus;
    const int64_t per_wg = (items + grid - 1) / grid;
    const int64_t smem =
        2 * DW * (int64_t)buf_bytes + (WK > 1 ? per_wg * DRG * WK * MR * 4 : 0);
    if (smem > 65536 - 64) return hipErrorNotSupported;
    const int Kp = (int)((K + 255) / 256 * 256);
    for (int64_t m0 = 0; m0 < M; m0 += MR) {
        const int mc = (int)(M - m0 < MR ? M - m0 : MR);
        launch_kernel((k_gemv_dyn<FMT, 1, WK, NL, false, false, false, MR>),
                      dim3((unsigned)grid), dim3(DWG), (unsigned)smem, st, (const uint8_t*)w,
                      (int)N, U, g.US, (int)(K / 32), row_bytes_of(FMT, K), buf_bytes,
                      q + m0 * Kp, d + m0 * (Kp / 32), s + m0 * (Kp / 32), y + m0 * N,
                      SwigluOut{}, ActIn{}, Kp, mc);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int FMT, int MR>
hipError_t launch_rows_mr(const void* w, int64_t N, int64_t K, int64_t M, const int8_t* q,
                          const uint16_t* d, const int32_t* s, float* y, hipStream_t st) {
    // the split-K of the batch-1 streaming kernels (same slices, same bits)
    const int U = units_of(FMT, K);
    if (U > 256) return hipErrorNotSupported;
    if (U > 128) return launch_rows_cfg<FMT, 4, MR>(w, N, K, M, q, d, s, y, st);
    if (U > 64) return launch_rows_cfg<FMT, 2, MR>(w, N, K, M, q, d, s, y, st);
    return launch_rows_cfg<FMT, 1, MR>(w, N, K, M, q, d, s, y, st);
}

template <int FMT>
hipError_t launch_rows_fmt(const void* w, int64_t N, int64_t K, int64_t M, const int8_t* q,
                           const uint16_t* d, const int32_t* s, float* y, hipStream_t st) {
    if (M == 2) return launch_rows_mr<FMT, 2>(w, N, K, M, q, d, s, y, st);
    return launch_rows_mr<FMT, 4>(w, N, K, M, q, d, s, y, st);
}

}  // namespace

hipError_t launch_small_m_rows(int fmt, const void* w, int64_t N, int64_t K, int64_t M,
                               const int8_t* q, const uint16_t* d, const int32_t* s, float* y,
                               hipStream_t st) {
    switch (fmt) {
    case QGEMV_FMT_Q4_K: return launch_rows_fmt<QGEMV_FMT_Q4_K>(w, N, K, M, q, d, s, y, st);
    case QGEMV_FMT_Q6_K: return launch_rows_fmt<QGEMV_FMT_Q6_K>(w, N, K, M, q, d, s, y, st);
    case QGEMV_FMT_Q4_0: return launch_rows_fmt<QGEMV_FMT_Q4_0>(w, N, K, M, q, d, s, y, st);
    default: return hipErrorNotSupported;
    }
}

}  // namespace qgemv
