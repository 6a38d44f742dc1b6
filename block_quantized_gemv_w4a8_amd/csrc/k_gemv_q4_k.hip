// k_gemv_q4_k.hip -- the Q4_K GEMV launchers (kernel templates in k_gemv.h).
#include "k_gemv.h"

namespace qgemv {

QGEMV_GEMV_FORMAT_ENTRIES(q4_k, QGEMV_FMT_Q4_K)
// The fused gate|up product always takes the LDS-streaming kernel (with the
// split-K of launch_gemv_fmt); every Q4_K row up to QGEMV_K_MAX fits its
// slice buffers, and its activation row too when the kernel forms it.
hipError_t launch_q4k_swiglu(const GemvArgs& a, const SwigluOut& so, hipStream_t st) {
    constexpr int FMT = QGEMV_FMT_Q4_K;
    const int U = units_of(FMT, a.K);
    const SliceGeom g = slice_geom<FMT>(a.K, U, lds_wk<FMT>(U));
    if (!lds_slice_fits<FMT>(g)) return hipErrorInvalidValue;
    return launch_lds_fmt<FMT, true, false>(a, U, g, st, so, {});
}

hipError_t launch_quantize_q4k_swiglu(const GemvArgs& a, const SwigluOut& so, const ActIn& ai,
                                      hipStream_t st) {
    constexpr int FMT = QGEMV_FMT_Q4_K;
    const int U = units_of(FMT, a.K);
    const int Kp = (int)((a.K + 255) / 256 * 256);
    const SliceGeom g = slice_geom<FMT>(a.K, U, lds_wk<FMT>(U));
    if (!lds_slice_fits<FMT>(g, act_lds_bytes(Kp))) return hipErrorInvalidValue;
    return launch_lds_fmt<FMT, true, true>(a, U, g, st, so, ai);
}

}  // namespace qgemv
