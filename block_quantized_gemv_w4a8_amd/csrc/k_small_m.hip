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
// the fp32 MFMA (v_mfma_f32_16x16x4f32) instead of the vector ALUs.  Weights
// and activation are staged through LDS with coalesced 16-byte loads, and
// the eight sub-blocks of a super-block are split between two waves.
#include <type_traits>

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

// Geometry of the MFMA variant.  A workgroup owns ROWS = 16*RT weight rows
// and all MP = 16*MT activation rows, and walks K in steps of G super-blocks.
// One step of its weights and activation sits in LDS (double-buffered):
//   weights:    ROWS rows x (G*144 bytes + 16 pad), the row's G super-blocks
//               as they lie in HBM
//   activation: G x { codes [MP][256 + 16 pad], fp32 dx [8][MP], dx*s [8][MP] }
// The pads put the 16 rows a wave reads at once on different LDS banks.
template <int MT, int RT, int G>
struct MfmaGeom {
    static constexpr int MP = 16 * MT;
    static constexpr int ROWS = 16 * RT;
    static constexpr int WSTRIDE = 144 * G + 16;
    static constexpr int WBYTES = ROWS * WSTRIDE;
    static constexpr int ASTRIDE = 272;
    static constexpr int ACODES = MP * ASTRIDE;
    static constexpr int ASTAGE = ACODES + 2 * 8 * MP * 4;
    static constexpr int BUF = WBYTES + G * ASTAGE;
};

// Wave (rt, part) of the workgroup computes weight tile rt (rows 16*rt ..
// 16*rt + 15) over sub-blocks part*BPW .. part*BPW + BPW-1 of every
// super-block (BPW = 8/KS); the KS partial sums of a tile are added in LDS
// at the end, always in part order.  Lane l: weight row 16*rt + l%16, K part
// 8*(l/16) of each 32-block (the i8 MFMA operand layout); its outputs are
// rows 16t + 4*(l/16) + i of that weight row.
//
// The weights are read from HBM the way the GEMV reads them: each lane loads
// 16 consecutive bytes and a wave instruction covers about 1 KB of
// consecutive row bytes, so whole cache lines are used by one instruction.
// (Loading the MFMA operand layout straight from HBM -- 16 rows x 8 bytes per
// instruction -- costs several cache-line requests per 144-byte super-block
// and leaves the kernel waiting on them.)
template <int MT, int RT, int KS, int G, int R>
__global__ __launch_bounds__(64 * RT * KS) void k_small_m_mfma(const uint8_t* __restrict__ w,
                                                               int N, int Kp, int M,
                                                               const int8_t* __restrict__ q,
                                                               const uint16_t* __restrict__ d,
                                                               const int32_t* __restrict__ s,
                                                               float* __restrict__ y) {
    static_assert(KS == 1 || KS == 2 || KS == 4, "sub-blocks split over 1, 2 or 4 waves");
    using GM = MfmaGeom<MT, RT, G>;
    constexpr int MP = GM::MP, ROWS = GM::ROWS;
    constexpr int NT = 64 * RT * KS;                         // threads
    constexpr int BPW = 8 / KS;                              // sub-blocks per wave and super-block
    constexpr int WCH = ROWS * 9 * G;                        // 16-byte weight chunks per step
    constexpr int WPT = (WCH + NT - 1) / NT;
    constexpr int ACH = G * MP * 16;                         // 16-byte code chunks per step
    constexpr int APT = (ACH + NT - 1) / NT;
    constexpr int SCH = G * 8 * MP;                          // scale entries per step
    constexpr int SPT = (SCH + NT - 1) / NT;
    constexpr int PART_BYTES = (KS - 1) * RT * MT * 4 * 64 * 4;
    constexpr int SMEM = 2 * GM::BUF > PART_BYTES ? 2 * GM::BUF : PART_BYTES;
    __shared__ __align__(16) uint8_t smem[SMEM];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rt = wave % RT, part = wave / RT;
    const int nl = lane & 15, kp = lane >> 4;
    const int row0 = blockIdx.x * ROWS;
    const int n = row0 + 16 * rt + nl;
    const int nsb = Kp / 256, nb = Kp / 32;
    const int nsteps = (nsb + G - 1) / G;
    const int64_t row_bytes = (int64_t)nsb * Q4K::SB_BYTES;

    // One step's global data in registers between load and LDS store.  Every
    // load is issued unconditionally with its address clamped into the
    // buffers (rows past N re-read row N-1, super-blocks past K re-read the
    // last one, activation rows past M re-read row M-1; none of those reach
    // a stored output): a load behind a branch makes the compiler drain all
    // outstanding loads.
    struct Regs {
        u32x4 wc[WPT];
        u32x4 ac[APT];
        uint32_t dh[SPT];
        int32_t sv[SPT];
    };
    auto load_step = [&](int st, Regs& r) {
#pragma unroll
        for (int k = 0; k < WPT; k++) {
            const int c = min(tid + NT * k, WCH - 1);
            const int row = c / (9 * G), off = c - row * (9 * G);
            const int sb = min(G * st + off / 9, nsb - 1);
            const uint8_t* p = w + (int64_t)min(row0 + row, N - 1) * row_bytes +
                               Q4K::SB_BYTES * sb + 16 * (off % 9);
            r.wc[k] = *reinterpret_cast<const u32x4*>(p);
        }
#pragma unroll
        for (int k = 0; k < APT; k++) {
            const int c = min(tid + NT * k, ACH - 1);
            const int g = c / (MP * 16), rem = c - g * (MP * 16);
            const int m = min(rem >> 4, M - 1), cc = rem & 15;
            const int sb = min(G * st + g, nsb - 1);
            r.ac[k] = *reinterpret_cast<const u32x4*>(q + (int64_t)m * Kp + 256 * sb + 16 * cc);
        }
#pragma unroll
        for (int k = 0; k < SPT; k++) {
            const int c = min(tid + NT * k, SCH - 1);
            const int g = c / (8 * MP), rem = c - g * (8 * MP);
            const int j = rem / MP, m = min(rem - j * MP, M - 1);
            const int sb = min(G * st + g, nsb - 1);
            const int64_t b = (int64_t)m * nb + 8 * sb + j;
            r.dh[k] = d[b];
            r.sv[k] = s[b];
        }
    };
    auto store_step = [&](const Regs& r, int buf) {
        uint8_t* base = smem + buf * GM::BUF;
#pragma unroll
        for (int k = 0; k < WPT; k++) {
            const int c = tid + NT * k;
            if (c < WCH) {
                const int row = c / (9 * G), off = c - row * (9 * G);
                *reinterpret_cast<u32x4*>(base + row * GM::WSTRIDE + 16 * off) = r.wc[k];
            }
        }
        uint8_t* act = base + GM::WBYTES;
#pragma unroll
        for (int k = 0; k < APT; k++) {
            const int c = tid + NT * k;
            if (c < ACH) {
                const int g = c / (MP * 16), rem = c - g * (MP * 16);
                *reinterpret_cast<u32x4*>(act + g * GM::ASTAGE + (rem >> 4) * GM::ASTRIDE +
                                          16 * (rem & 15)) = r.ac[k];
            }
        }
#pragma unroll
        for (int k = 0; k < SPT; k++) {
            const int c = tid + NT * k;
            if (c < SCH) {
                const int g = c / (8 * MP), rem = c - g * (8 * MP);   // rem = j * MP + m
                float* dx = reinterpret_cast<float*>(act + g * GM::ASTAGE + GM::ACODES);
                const float f = h2f(r.dh[k]);
                dx[rem] = f;
                dx[8 * MP + rem] = f * (float)r.sv[k];
            }
        }
    };

    // one accumulator set per super-block of a step (G independent chains),
    // or a single set where MT is large and registers are short
    constexpr int AG = MT >= 3 ? 1 : G;
    f32x4 acc[AG][MT], acc2[AG][MT];
#pragma unroll
    for (int g = 0; g < AG; g++)
#pragma unroll
        for (int t = 0; t < MT; t++) {
            acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc2[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    const i32x4 zero = {0, 0, 0, 0};

    // Super-block g of the step in LDS buffer buf, for part P of the
    // sub-blocks (P is the wave's part as a compile-time constant, so the
    // scale bytes and LDS offsets of its sub-blocks are constants too).
    // With PIN set (large MT) empty volatile asm statements make the MFMAs of
    // sub-block jj+1 go out before the scaling of jj and keep every other
    // sub-block in order; without them the compiler issues all the MFMAs
    // first and holds all their results in registers.  At small MT it may.
    // A super-block past the end of K (the tail of the last step) holds a
    // copy of the last one; its scales are taken as zero, so it adds exact
    // zeros.
    auto compute_sb = [&](auto Pc, auto Gc, int buf, bool valid) {
        constexpr int P = decltype(Pc)::value;
        constexpr int g = decltype(Gc)::value;
        constexpr int ga = g < AG ? g : AG - 1;   // accumulator set
        constexpr bool PIN = MT >= 3;
        const int ow = buf * GM::BUF + (16 * rt + nl) * GM::WSTRIDE + Q4K::SB_BYTES * g;
        const u32x4 hdr = *reinterpret_cast<const u32x4*>(smem + ow);
        const float fd = valid ? h2f(hdr.x & 0xFFFFu) : 0.0f;
        const float fdm = valid ? h2f(hdr.x >> 16) : 0.0f;
        // 6-bit scales of sub-blocks 0..3 (bytes of hdr.y) and 4..7 (low
        // nibbles of hdr.w, high bits from the top of hdr.y), four per dword
        const uint32_t slo = hdr.y & 0x3F3F3F3Fu;
        const uint32_t shi = (hdr.w & LO4) | ((hdr.y >> 2) & 0x30303030u);
        const int oa = buf * GM::BUF + GM::WBYTES + g * GM::ASTAGE;
        auto mfma_block = [&](int jj, i32x4 (&D)[MT]) {
            const int j = P * BPW + jj;
            int o = ow + 16 + 32 * (j >> 1) + 8 * kp;
            int o2 = oa + 32 * j;
            if (PIN) asm volatile("" : "+v"(o), "+s"(o2));
            const u32x2 v = *reinterpret_cast<const u32x2*>(smem + o);
            const int sh = 4 * (j & 1);
            const long B = (long)(((uint64_t)((v.y >> sh) & LO4) << 32) | ((v.x >> sh) & LO4));
#pragma unroll
            for (int t = 0; t < MT; t++) {
                const long A = *reinterpret_cast<const long*>(
                    smem + o2 + (16 * t + nl) * GM::ASTRIDE + 8 * kp);
                D[t] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B, zero, 0, 0, 0);
            }
        };
        auto scale_block = [&](int jj, const i32x4 (&D)[MT]) {
            const int j = P * BPW + jj;
            const float wsj = fd * (float)(((j >= 4 ? shi : slo) >> (8 * (j & 3))) & 0xFFu);
            int o = oa + GM::ACODES + 4 * j * MP;
            if (PIN) asm volatile("" : "+s"(o));
#pragma unroll
            for (int t = 0; t < MT; t++) {
                const f32x4 x4 = *reinterpret_cast<const f32x4*>(smem + o + 4 * (16 * t + 4 * kp));
#pragma unroll
                for (int i = 0; i < 4; i++)
                    acc[ga][t][i] = fmaf((float)D[t][i], wsj * x4[i], acc[ga][t][i]);
            }
            if (PIN) {
#pragma unroll
                for (int t = 0; t < MT; t++) asm volatile("" : "+v"(acc[ga][t]));
            }
        };
        i32x4 D2[2][MT];
        mfma_block(0, D2[0]);
#pragma unroll
        for (int jj = 1; jj < BPW; jj++) {
            mfma_block(jj, D2[jj & 1]);
            scale_block(jj - 1, D2[(jj - 1) & 1]);
        }
        scale_block(BPW - 1, D2[(BPW - 1) & 1]);
        // min term: rows m x sub-blocks j (dx*s) times sub-blocks j x this
        // lane's row (dmin*m_j); MFMA K lane kp carries sub-block 4*kk + kp,
        // and lanes whose sub-block belongs to another wave contribute zero.
        // The 6-bit mins: bytes of hdr.z (sub-blocks 0..3), or high nibbles
        // of hdr.w with high bits from the top of hdr.z (4..7).
        const uint32_t mlo = hdr.z & 0x3F3F3F3Fu;
        const uint32_t mhi = ((hdr.w >> 4) & LO4) | ((hdr.z >> 2) & 0x30303030u);
        const float* dxs = reinterpret_cast<const float*>(smem + oa + GM::ACODES + 4 * 8 * MP);
#pragma unroll
        for (int kk = 0; kk < (BPW == 8 ? 2 : 1); kk++) {
            constexpr int JB = BPW == 8 ? 0 : (P * BPW) & ~3;   // first sub-block of the group
            const int jg = BPW == 8 ? 4 * kk : JB;
            const bool mine = BPW >= 4 || (kp >> 1) == (P & 1);
            const uint32_t mb = jg >= 4 ? mhi : mlo;
            const float b = mine ? fdm * (float)bfe(mb, 8 * kp, 8) : 0.0f;
#pragma unroll
            for (int t = 0; t < MT; t++) {
                const float a = dxs[(jg + kp) * MP + 16 * t + nl];
                acc2[ga][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc2[ga][t], 0, 0, 0);
            }
        }
    };
    auto compute_part = [&](auto Pc, int buf, int st) {
        compute_sb(Pc, std::integral_constant<int, 0>{}, buf, true);
        if (G > 1) compute_sb(Pc, std::integral_constant<int, (G > 1 ? 1 : 0)>{}, buf, G * st + 1 < nsb);
        static_assert(G <= 2, "one or two super-blocks per step");
    };
    auto compute_step = [&](int buf, int st) {
        if (KS == 1) {
            compute_part(std::integral_constant<int, 0>{}, buf, st);
        } else if (KS == 2) {
            if (part == 0) compute_part(std::integral_constant<int, 0>{}, buf, st);
            else compute_part(std::integral_constant<int, 1>{}, buf, st);
        } else {
            switch (part) {
            case 0: compute_part(std::integral_constant<int, 0>{}, buf, st); break;
            case 1: compute_part(std::integral_constant<int, 1>{}, buf, st); break;
            case 2: compute_part(std::integral_constant<int, 2>{}, buf, st); break;
            default: compute_part(std::integral_constant<int, 3>{}, buf, st); break;
            }
        }
    };

    // Software pipeline over steps, R deep: step st issues the global loads
    // of step st+R into register set st mod R, computes st from LDS buffer
    // st&1, and stores step st+1 (loaded R-1 steps earlier) into the other
    // buffer.  It starts at st = -R with nothing loaded, and every step
    // issues the same loads, so the compiler's wait counts stay exact.
    Regs rg[R];
    for (int base = -R; base < nsteps; base += R) {
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int st = base + r;
            load_step(min(st + R, nsteps - 1), rg[r]);
            __builtin_amdgcn_sched_barrier(0);
            if (st >= 0 && st < nsteps) compute_step(st & 1, st);
            if (st + 1 >= 0 && st + 1 < nsteps) store_step(rg[(r + 1) % R], (st + 1) & 1);
            __syncthreads();
        }
    }

    // partial sums of parts 1 .. KS-1 go through LDS (free after the last
    // step's barrier); part 0 adds them in part order and stores
    float* pbuf = reinterpret_cast<float*>(smem);
    auto partial = [&](int t, int i) {
        float v = acc[0][t][i] - acc2[0][t][i];
#pragma unroll
        for (int g = 1; g < AG; g++) v += acc[g][t][i] - acc2[g][t][i];
        return v;
    };
    auto pidx = [&](int p, int t, int i) {
        return (((p - 1) * RT + rt) * MT * 4 + 4 * t + i) * 64 + lane;
    };
    if (KS > 1 && part > 0) {
#pragma unroll
        for (int t = 0; t < MT; t++)
#pragma unroll
            for (int i = 0; i < 4; i++) pbuf[pidx(part, t, i)] = partial(t, i);
    }
    if (KS > 1) __syncthreads();
    if (part == 0 && n < N) {
#pragma unroll
        for (int t = 0; t < MT; t++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                float v = partial(t, i);
#pragma unroll
                for (int p = 1; p < KS; p++) v += pbuf[pidx(p, t, i)];
                const int m = 16 * t + 4 * kp + i;
                if (m < M) y[(int64_t)m * N + n] = v;
            }
    }
}

// Waves sharing one weight tile's sub-blocks.  Fixed for every M, so row m of
// a product does not depend on the other rows in the batch.
constexpr int kMfmaSplit = 2;
// Super-blocks per step.
constexpr int kMfmaStep = 2;

// RT: weight tiles per workgroup (the activation staged by a workgroup is
// shared by 16*RT weight rows); R: steps of global loads in flight.
template <int MT, int RT, int R>
static hipError_t launch_mfma_mt(const void* w, int64_t N, int64_t K, int64_t M,
                                 const int8_t* q, const uint16_t* d, const int32_t* s, float* y,
                                 hipStream_t st) {
    const int Kp = (int)((K + 255) / 256 * 256);
    const int64_t grid = (N + 16 * RT - 1) / (16 * RT);
    hipLaunchKernelGGL((k_small_m_mfma<MT, RT, kMfmaSplit, kMfmaStep, R>), dim3((unsigned)grid),
                       dim3(64 * RT * kMfmaSplit), 0, st, (const uint8_t*)w, (int)N, Kp, (int)M,
                       q, d, s, y);
    return hipGetLastError();
}

static hipError_t launch_mfma(const void* w, int64_t N, int64_t K, int64_t M, const int8_t* q,
                              const uint16_t* d, const int32_t* s, float* y, hipStream_t st) {
    const int mt = (int)((M + 15) / 16);
    switch (mt) {
    case 1: return launch_mfma_mt<1, 2, 2>(w, N, K, M, q, d, s, y, st);
    case 2: return launch_mfma_mt<2, 4, 2>(w, N, K, M, q, d, s, y, st);
    case 3: return launch_mfma_mt<3, 4, 2>(w, N, K, M, q, d, s, y, st);
    default: return launch_mfma_mt<4, 4, 2>(w, N, K, M, q, d, s, y, st);
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
constexpr int kMfmaFromM = 3;

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
