// k_small_m.hip -- a few activation rows (the prefill chunk) against Q4_K
// weights.  Output row m equals the batch-1 GEMV of activation row m (colibri
// GPU backends, eligibility gates: C = A x B is row-independent).
//
// DOT4 variant: the GEMV kernel's mapping (LPR lanes per weight row, one
// 64-weight unit per lane step), except that each weight unit is loaded and
// unpacked once and then dotted against MT activation rows staged in LDS, so
// the weight stream is shared by the MT rows ("Backends and hardware",
// section "CUDA": W4A8 inner product on 4 x int8 dots).
//
// MFMA variant: where the work is a dense contraction (many rows), the int8
// matrix cores do it.  Each 32-wide K block gets its own int8 MFMA
// (v_mfma_i32_16x16x32_i8: a 16 x 16 tile of exact int32 block dots), because
// both sides carry a scale per 32-block; the fp32 epilogue then adds
// D * (d * sc_j) * dx per tile element.  The min term
// sum_b (dmin * m_j) * (dx * s) is itself a small dense product and goes to
// the fp32 MFMA (v_mfma_f32_16x16x4f32) instead of the vector ALUs.
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

// ----------------------------------------------------------------- MFMA --

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// LDS of one K stage (one super-block, 256 columns) for all MP = 16*MT rows:
// codes [MP][ACT_STRIDE] (rows padded by 16 bytes against bank conflicts),
// then fp32 dx [8][MP] and dx*s [8][MP] (block j of the super-block, row m).
template <int MT>
struct MfmaStage {
    static constexpr int MP = 16 * MT;
    static constexpr int ACT_STRIDE = 272;
    static constexpr int CODES = MP * ACT_STRIDE;
    static constexpr int BYTES = CODES + 2 * 8 * MP * 4;
};

// One wave = one 16-row weight tile (rows n0 .. n0+15) x all MP activation
// rows x all of K.  Lane l: weight row n0 + l%16, K part 8*(l/16) of each
// 32-block (the i8 MFMA operand layout); its outputs are rows
// 16t + 4*(l/16) + i, column n0 + l%16.  The NW waves of a workgroup share
// the activation, staged per super-block in LDS (double-buffered); the next
// super-block's activation is loaded into registers before the current one
// is computed and written to LDS after it, and each lane's weights run three
// super-blocks ahead in a register ring, so the loads overlap the math.
template <int MT, int NW>
__global__ __launch_bounds__(64 * NW) void k_small_m_mfma(const uint8_t* __restrict__ w, int N,
                                                          int Kp, int M,
                                                          const int8_t* __restrict__ q,
                                                          const uint16_t* __restrict__ d,
                                                          const int32_t* __restrict__ s,
                                                          float* __restrict__ y) {
    using SG = MfmaStage<MT>;
    constexpr int MP = SG::MP;
    constexpr int NT = 64 * NW;                       // threads
    constexpr int CPT = (MP * 16 + NT - 1) / NT;      // 16-byte code chunks per thread
    constexpr int SPT = (8 * MP + NT - 1) / NT;       // scale entries per thread
    __shared__ __align__(16) uint8_t smem[2 * SG::BYTES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nl = lane & 15, kp = lane >> 4;
    const int n = (blockIdx.x * NW + wave) * 16 + nl;
    const int nsb = Kp / 256, nb = Kp / 32;
    const uint8_t* wrow = w + (int64_t)min(n, N - 1) * (nsb * Q4K::SB_BYTES);

    // activation of super-block S held in registers between load and store
    struct ActRegs {
        u32x4 c[CPT];
        uint32_t dh[SPT];
        int32_t sv[SPT];
    };
    auto load_act = [&](int S, ActRegs& r) {
#pragma unroll
        for (int k = 0; k < CPT; k++) {
            const int i = tid + NT * k;
            const int m = i >> 4, c = i & 15;
            r.c[k] = u32x4{0u, 0u, 0u, 0u};
            if (i < MP * 16 && m < M)
                r.c[k] = *reinterpret_cast<const u32x4*>(q + (int64_t)m * Kp + 256 * S + 16 * c);
        }
#pragma unroll
        for (int k = 0; k < SPT; k++) {
            const int i = tid + NT * k;
            const int j = i / MP, m = i - j * MP;
            r.dh[k] = 0u;
            r.sv[k] = 0;
            if (i < 8 * MP && m < M) {
                const int64_t b = (int64_t)m * nb + 8 * S + j;
                r.dh[k] = d[b];
                r.sv[k] = s[b];
            }
        }
    };
    auto store_act = [&](const ActRegs& r, int buf) {
        uint8_t* base = smem + buf * SG::BYTES;
#pragma unroll
        for (int k = 0; k < CPT; k++) {
            const int i = tid + NT * k;
            if (i < MP * 16)
                *reinterpret_cast<u32x4*>(base + (i >> 4) * SG::ACT_STRIDE + 16 * (i & 15)) = r.c[k];
        }
        float* dx = reinterpret_cast<float*>(base + SG::CODES);
#pragma unroll
        for (int k = 0; k < SPT; k++) {
            const int i = tid + NT * k;
            if (i < 8 * MP) {
                const float f = h2f(r.dh[k]);
                dx[i] = f;                       // [j][m]: i = j * MP + m
                dx[8 * MP + i] = f * (float)r.sv[k];
            }
        }
    };
    // this lane's weights of super-block S: header and 4 x 8 code bytes
    struct WQ {
        u32x4 hdr;
        u32x2 qs[4];
    };
    auto load_w = [&](int S, WQ& wq) {
        const uint8_t* p = wrow + Q4K::SB_BYTES * min(S, nsb - 1);
        wq.hdr = ld16(p);
#pragma unroll
        for (int c = 0; c < 4; c++) wq.qs[c] = ld8(p + 16 + 32 * c + 8 * kp);
    };

    f32x4 acc[MT], acc2[MT];
#pragma unroll
    for (int t = 0; t < MT; t++) {
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc2[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const i32x4 zero = {0, 0, 0, 0};

    auto compute = [&](int buf, const WQ& wq) {
        const uint8_t* base = smem + buf * SG::BYTES;
        const float* dx = reinterpret_cast<const float*>(base + SG::CODES);
        const float* dxs = dx + 8 * MP;
        Q4K::W hw;
        hw.hdr = wq.hdr;
        const float fd = h2f(wq.hdr.x & 0xFFFFu), fdm = h2f(wq.hdr.x >> 16);
#pragma unroll
        for (int c = 0; c < 4; c++) {
#pragma unroll
            for (int hbit = 0; hbit < 2; hbit++) {
                const int j = 2 * c + hbit;
                int sc, mn;
                Q4K::scale_min(hw, j, sc, mn);
                const float wsj = fd * (float)sc;
                const uint32_t b0 = hbit ? (wq.qs[c].x >> 4) & LO4 : wq.qs[c].x & LO4;
                const uint32_t b1 = hbit ? (wq.qs[c].y >> 4) & LO4 : wq.qs[c].y & LO4;
                const long B = (long)(((uint64_t)b1 << 32) | b0);
#pragma unroll
                for (int t = 0; t < MT; t++) {
                    const long A = *reinterpret_cast<const long*>(
                        base + (16 * t + nl) * SG::ACT_STRIDE + 32 * j + 8 * kp);
                    const i32x4 D = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B, zero, 0, 0, 0);
                    const f32x4 x4 = *reinterpret_cast<const f32x4*>(dx + j * MP + 16 * t + 4 * kp);
#pragma unroll
                    for (int i = 0; i < 4; i++) acc[t][i] = fmaf((float)D[i], wsj * x4[i], acc[t][i]);
                }
                // one 32-block at a time: keeps the MFMA results and their
                // operands from piling up in registers
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // min term: rows m x blocks j (dx*s) times blocks j x this lane's row n (dmin*m_j)
#pragma unroll
        for (int kk = 0; kk < 2; kk++) {
            int sc, mn;
            Q4K::scale_min(hw, 4 * kk + kp, sc, mn);
            const float b = fdm * (float)mn;
#pragma unroll
            for (int t = 0; t < MT; t++) {
                const float a = dxs[(4 * kk + kp) * MP + 16 * t + nl];
                acc2[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc2[t], 0, 0, 0);
            }
        }
    };

    // one super-block: load the activation of S+1, compute S from its ring
    // slot, refill the slot with the weights of S+3, publish the activation
    ActRegs ar;
    auto step = [&](int S, WQ& slot) {
        if (S + 1 < nsb) load_act(S + 1, ar);
        __builtin_amdgcn_sched_barrier(0);
        compute(S & 1, slot);
        load_w(S + 3, slot);
        if (S + 1 < nsb) store_act(ar, (S + 1) & 1);
        __syncthreads();
    };

    WQ w0, w1, w2;
    load_w(0, w0);
    load_w(1, w1);
    load_w(2, w2);
    load_act(0, ar);
    store_act(ar, 0);
    __syncthreads();
    for (int S = 0; S < nsb; S += 3) {
        step(S, w0);
        if (S + 1 < nsb) step(S + 1, w1);
        if (S + 2 < nsb) step(S + 2, w2);
    }
    if (n < N) {
#pragma unroll
        for (int t = 0; t < MT; t++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int m = 16 * t + 4 * kp + i;
                if (m < M) y[(int64_t)m * N + n] = acc[t][i] - acc2[t][i];
            }
    }
}

template <int MT, int NW>
static hipError_t launch_mfma_mt(const void* w, int64_t N, int64_t K, int64_t M,
                                 const int8_t* q, const uint16_t* d, const int32_t* s, float* y,
                                 hipStream_t st) {
    const int Kp = (int)((K + 255) / 256 * 256);
    const int64_t grid = (N + 16 * NW - 1) / (16 * NW);
    hipLaunchKernelGGL((k_small_m_mfma<MT, NW>), dim3((unsigned)grid), dim3(64 * NW), 0, st,
                       (const uint8_t*)w, (int)N, Kp, (int)M, q, d, s, y);
    return hipGetLastError();
}

// Waves (16-row weight tiles) per workgroup of the MFMA variant.
constexpr int kMfmaWaves = 4;

static hipError_t launch_mfma(const void* w, int64_t N, int64_t K, int64_t M, const int8_t* q,
                              const uint16_t* d, const int32_t* s, float* y, hipStream_t st) {
    const int mt = (int)((M + 15) / 16);
    switch (mt) {
    case 1: return launch_mfma_mt<1, kMfmaWaves>(w, N, K, M, q, d, s, y, st);
    case 2: return launch_mfma_mt<2, kMfmaWaves>(w, N, K, M, q, d, s, y, st);
    case 3: return launch_mfma_mt<3, kMfmaWaves>(w, N, K, M, q, d, s, y, st);
    default: return launch_mfma_mt<4, kMfmaWaves>(w, N, K, M, q, d, s, y, st);
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

// AUTO: the MFMA variant from this many rows on (measured crossover).
constexpr int kMfmaFromM = 2;

hipError_t launch_small_m_q4k(const void* w, int64_t N, int64_t K, int64_t M, const int8_t* q,
                              const uint16_t* d, const int32_t* s, float* y, int variant,
                              hipStream_t st) {
    if (variant == QGEMV_VARIANT_MFMA || (variant == QGEMV_VARIANT_AUTO && M >= kMfmaFromM))
        return launch_mfma(w, N, K, M, q, d, s, y, st);
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
