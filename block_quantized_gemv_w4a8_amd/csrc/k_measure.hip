// k_measure.hip -- a measurement aid: a plain streaming read of a device
// buffer with 16-byte loads, the achievable HBM read rate that the GEMV
// kernels are compared with (the decode step is bound by streaming the
// weights: "Running an LLM on VKNN", Performance).  Nothing in the GEMV path
// uses it.
#include "qgemv_device.h"
#include "qgemv_launch.h"

namespace qgemv {

constexpr int RWG = 256;    // threads per workgroup
constexpr int RUNROLL = 8;  // 16-byte loads in flight per thread

// Every thread reads RUNROLL chunks of 16 bytes per pass, a workgroup 32 KB
// of consecutive bytes, the grid striding over the buffer; indices past the
// end are clamped to the last chunk (re-read from cache, no branch around
// the loads).  The loaded words are folded into one value that is stored
// only when it equals a constant, so the loads cannot be dropped and
// (practically) nothing is written.
template <bool NT>
__global__ __launch_bounds__(RWG) void k_stream_read(const u32x4* __restrict__ p, int64_t n16,
                                                     uint32_t* __restrict__ sink) {
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * RWG * RUNROLL;
    for (int64_t base = (int64_t)blockIdx.x * RWG * RUNROLL + threadIdx.x; base < n16;
         base += stride) {
        u32x4 v[RUNROLL];
#pragma unroll
        for (int u = 0; u < RUNROLL; u++) {
            const u32x4* a = p + min(base + (int64_t)u * RWG, n16 - 1);
            v[u] = NT ? __builtin_nontemporal_load(a) : *a;
        }
#pragma unroll
        for (int u = 0; u < RUNROLL; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

hipError_t launch_stream_read(const void* buf, int64_t bytes, int nontemporal, uint32_t* sink,
                              int wg_per_cu, hipStream_t st) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0) {
        (void)hipGetLastError();
        cus = 256;
    }
    const int64_t n16 = bytes / 16;
    const int64_t per_pass = (int64_t)RWG * RUNROLL;
    int64_t grid = (int64_t)cus * wg_per_cu;
    const int64_t need = (n16 + per_pass - 1) / per_pass;
    if (grid > need) grid = need;
    if (nontemporal)
        launch_kernel(k_stream_read<true>, dim3((unsigned)grid), dim3(RWG), 0, st,
                      (const u32x4*)buf, n16, sink);
    else
        launch_kernel(k_stream_read<false>, dim3((unsigned)grid), dim3(RWG), 0, st,
                      (const u32x4*)buf, n16, sink);
    return hipGetLastError();
}

}  // namespace qgemv
