// k_small_m.hip -- a few activation rows (the prefill chunk) against Q4_K,
// Q6_K or Q4_0 weights.  Output row m equals the batch-1 GEMV of activation
// row m (colibri GPU backends, eligibility gates: C = A x B is
// row-independent).
//
// DOT4 variant: one activation row is the batch-1 GEMV; more go through the
// batch-1 streaming kernel up to four at a time (k_small_m_rows.hip), each
// weight unit read once per group and dotted against every row of it with
// v_dot4 ("Backends and hardware", section "CUDA": W4A8 inner product on
// 4 x int8 dots).  Rows longer than that kernel takes (more than 256 units)
// fall back to k_small_m_dot4 below (Q4_K: the lanes-per-row mapping with
// each unit dotted against MT activation rows staged in LDS) or to the
// batch-1 GEMV on each row (Q6_K, Q4_0).
//
// MFMA variant (all three formats): where the work is a dense contraction
// (many rows), the int8 matrix cores do it.  Each 32-wide K block gets its
// own int8 MFMA (v_mfma_i32_16x16x32_i8: a 16 x 16 tile of exact int32 block
// dots; a Q6_K block takes two, one per 16-group), because both sides carry a
// scale per block; the fp32 epilogue then applies the weight and activation
// scales per tile element.  The remaining terms (the Q4_K min, the Q4_0 and
// Q6_K code offsets) are small dense products over the blocks and go to the
// fp32 MFMA (v_mfma_f32_16x16x4f32) instead of the vector ALUs.  Weights and
// activation are staged through LDS with coalesced 16-byte loads; the waves
// of a workgroup split the 32-blocks, the units of K and the activation tiles
// as the matrix shape and M call for.  Up to 8 activation rows a tile would
// be half padding; there one v_mfma_i32_16x16x64_i8 takes a pair of 32-blocks
// instead (tile rows 0-7 against the first block, 8-15 against the second,
// the other block's K lanes zeroed): the two-block tiles.
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

// Weight units of the MFMA variant: 256 consecutive weights of a row, which
// is a super-block of Q4_K (144 B) and Q6_K (210 B) and 8 blocks of Q4_0
// (8 x 18 = 144 B).  Q4_K units always start on 16-byte boundaries; Q6_K and
// Q4_0 units and rows only on 2-byte ones.
template <int FMT>
struct SmUnit;
template <>
struct SmUnit<QGEMV_FMT_Q4_K> {
    static constexpr int UB = 144;
    static constexpr bool ALIGNED = true;
    static constexpr bool S16 = false;   // per-16 activation sums needed
};
template <>
struct SmUnit<QGEMV_FMT_Q6_K> {
    static constexpr int UB = 210;
    static constexpr bool ALIGNED = false;
    static constexpr bool S16 = true;
};
template <>
struct SmUnit<QGEMV_FMT_Q4_0> {
    static constexpr int UB = 144;
    static constexpr bool ALIGNED = false;
    static constexpr bool S16 = false;
};

// LDS stride (bytes) of at least `need` whose dword count is 4 mod 8: the 16
// rows a wave reads at once then start on 16 different 4-bank groups.
constexpr int odd_quad_stride(int need) {
    int dw = (need + 3) / 4;
    while (dw % 8 != 4) dw++;
    return 4 * dw;
}

// Geometry of the MFMA variant.  A workgroup owns ROWS = 16*RT weight rows
// and all MP = 16*MT activation rows, and walks K in steps of G units.  One
// step of its weights and activation sits in LDS (double-buffered):
//   weights:    ROWS rows x WSTRIDE; a row holds the step's SPAN = G*UB bytes
//               as they lie in HBM (for unaligned formats starting at FRONT
//               + delta, delta = the span's offset from the 16-byte boundary
//               below it; the front pad takes a last chunk that was shifted
//               back to end at the row end)
//   activation: G x { codes [MP][256 + 16 pad], fp32 dx [8][MP], dx*s [8][MP]
//               (, int32 sums of each 16 codes [16][MP] for Q6_K) }
template <int FMT, int MT, int RT, int G>
struct MfmaGeom {
    using U = SmUnit<FMT>;
    static constexpr int MP = 16 * MT;
    static constexpr int ROWS = 16 * RT;
    static constexpr int SPAN = U::UB * G;
    static constexpr int NCH = U::ALIGNED ? SPAN / 16 : (SPAN + 14 + 15) / 16;
    static constexpr int FRONT = U::ALIGNED ? 0 : 16;
    static constexpr int WSTRIDE = U::ALIGNED ? SPAN + 16 : odd_quad_stride(FRONT + 16 * NCH + 16);
    static constexpr int WBYTES = ROWS * WSTRIDE;
    static constexpr int ASTRIDE = 272;
    static constexpr int ACODES = MP * ASTRIDE;
    static constexpr int ASCALE = 2 * 8 * MP * 4;
    static constexpr int ASTAGE = ACODES + ASCALE + (U::S16 ? 16 * MP * 4 : 0);
    static constexpr int BUF = WBYTES + G * ASTAGE;
};

// Wave (rt, ms, kq, ks) of the workgroup computes weight tile rt (rows
// 16*rt .. 16*rt + 15) against activation tiles ms*TPW .. ms*TPW + TPW-1
// (TPW = MT/MS tiles of 16 rows), over units kq, kq + KP, ... of every step
// and, within each, over 32-blocks ks*BPW .. ks*BPW + BPW-1 (BPW = 8/KS); the
// KS*KP partial sums of a tile are added in LDS at the end, always in the
// same order.  KP splits K between waves where the matrix has too few rows
// to fill the chip; MS splits the activation rows where M is large.  Lane l: weight row 16*rt + l%16, K part 8*(l/16) of
// each 32-block (the i8 MFMA operand layout); its outputs are rows
// 16t + 4*(l/16) + i of that weight row.
//
// The weights are read from HBM the way the GEMV reads them: each lane loads
// 16 consecutive bytes and a wave instruction covers about 1 KB of
// consecutive row bytes, so whole cache lines are used by one instruction.
// (Loading the MFMA operand layout straight from HBM -- 16 rows x 8 bytes per
// instruction -- costs several cache-line requests per 144-byte super-block
// and leaves the kernel waiting on them.)
//
// Per format, with D the 16 x 16 int32 tile of one 32-block (Q6_K: of one
// 16-group, the other half of the K lanes zeroed) and unsigned codes:
//   Q4_K  y += d*sc_j*dx*D  - (dmin*m_j)(dx*s)
//   Q4_0  y += dw*dx*D      - (8*dw)(dx*s)          (w = dw*(code - 8))
//   Q6_K  y += d*sc_g*dx*D  - (32*d*sc_g)(dx*sum16) (w = d*sc*(code - 32))
// The second product of each line is a small dense product over the blocks
// (groups) of a unit and goes to the fp32 MFMA.
//
// DOTS (validation): every int32 MFMA tile is also stored to dots [M][N][nb]
// (nb = Kp/32 blocks, Q4_0 K/32; Q6_K Kp/16 groups): the raw integer dots of
// the unsigned codes (Q4_K and Q4_0: sum code*q per 32-block; Q6_K: per
// 16-group) before any scale, offset or min is applied.
template <int FMT, int MT, int RT, int KS, int KP, int MS, int G, int R, bool DOTS = false,
          bool TWO = false>
__global__ __launch_bounds__(64 * RT * KS * KP * MS) void k_small_m_mfma(const uint8_t* __restrict__ w,
                                                               int N, int K, int Kp, int M,
                                                               const int8_t* __restrict__ q,
                                                               const uint16_t* __restrict__ d,
                                                               const int32_t* __restrict__ s,
                                                               float* __restrict__ y,
                                                               int32_t* __restrict__ dots) {
    static_assert(KS == 1 || KS == 2 || KS == 4, "32-blocks split over 1, 2 or 4 waves");
    static_assert(G % KP == 0 && (KP > 1 || G <= 2), "units of a step split evenly over KP");
    static_assert(MT % MS == 0, "activation tiles split evenly over MS");
    static_assert(!TWO || (MT == 1 && KS <= 4),
                  "two-block tiles: at most 8 activation rows, pairs of 32-blocks per wave");
    constexpr int TPW = MT / MS;                             // activation tiles per wave
    using GM = MfmaGeom<FMT, MT, RT, G>;
    using U = SmUnit<FMT>;
    constexpr int MP = GM::MP, ROWS = GM::ROWS, NCH = GM::NCH;
    constexpr int NT = 64 * RT * KS * KP * MS;               // threads
    constexpr int BPW = 8 / KS;                              // 32-blocks per wave and unit
    constexpr int WCH = ROWS * NCH;                          // 16-byte weight chunks per step
    constexpr int WPT = (WCH + NT - 1) / NT;
    constexpr int MA = TWO ? 8 : MP;                         // activation rows staged
    constexpr int ACH = G * MA * 16;                         // 16-byte code chunks per step
    constexpr int APT = (ACH + NT - 1) / NT;
    constexpr int SCH = G * 8 * MA;                          // scale entries per step
    constexpr int SPT = (SCH + NT - 1) / NT;
    constexpr int NPART = KS * KP;                           // partial sums per tile
    constexpr int PART_BYTES = (NPART - 1) * RT * MT * 4 * 64 * 4;
    constexpr int SMEM = 2 * GM::BUF > PART_BYTES ? 2 * GM::BUF : PART_BYTES;
    // two-block tiles, and Q6_K with one activation tile and whole units per
    // wave: 256 bytes of zeros after everything else, which the lanes whose
    // A-operand quarter belongs to the other block or to the other MFMA's
    // 16-group read instead of masking codes (Q6_K 12288 x 4096 at M = 16:
    // 23.5 against 24.0 us; with halved units, 4096 x 14336, 23.8 against
    // 23.3 us, so those keep the masks)
    constexpr bool ZA = TWO || (FMT == QGEMV_FMT_Q6_K && TPW == 1 && KS == 1);
    constexpr int ZOFF = SMEM, ZBYTES = ZA ? 256 : 0;
    __shared__ __align__(16) uint8_t smem[SMEM + ZBYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rt = wave % RT, ms = (wave / RT) % MS;
    const int part = wave / (RT * MS);                        // part = ks + KS * kq
    const int ks = part % KS, kq = part / KS;
    const int t0 = ms * TPW;                                  // first activation tile
    const int nl = lane & 15, kp = lane >> 4;
    const int row0 = blockIdx.x * ROWS;
    // activation rows: MP of them from m0 = MP * blockIdx.y (a second grid
    // dimension splits M between workgroups where whole tiles of weight rows
    // alone would leave compute units idle); the launch has M > m0
    {
        const int m0 = MP * blockIdx.y, nbk = Kp / 32;
        q += (int64_t)m0 * Kp;
        d += (int64_t)m0 * nbk;
        s += (int64_t)m0 * nbk;
        y += (int64_t)m0 * N;
        if constexpr (DOTS)
            dots += (int64_t)m0 * N *
                    (FMT == QGEMV_FMT_Q6_K ? 2 * nbk : (FMT == QGEMV_FMT_Q4_0 ? K / 32 : nbk));
        M = min(M - m0, MP);
    }
    if constexpr (ZA) {
        // (written before the pipeline's first barrier, read after it)
        if (tid < ZBYTES / 16) *reinterpret_cast<u32x4*>(smem + ZOFF + 16 * tid) = u32x4{0, 0, 0, 0};
    }
    const int n = row0 + 16 * rt + nl;
    const int nunits = Kp / 256, nb = Kp / 32;
    const int nbw = K / 32;                                  // weight blocks of a Q4_0 row
    const int nsteps = (nunits + G - 1) / G;
    const int64_t row_bytes = FMT == QGEMV_FMT_Q4_0 ? (int64_t)nbw * 18 : (int64_t)nunits * U::UB;
    const uint8_t* my_row = w + (int64_t)min(n, N - 1) * row_bytes;

    // 16-byte-aligned start of row r's span in step st, and the span's offset from it
    auto span_base = [&](const uint8_t* rowp, int st, int& delta) {
        const uint8_t* a = rowp + __umul24((unsigned)GM::SPAN, (unsigned)st);
        delta = (int)((uintptr_t)a & 15);
        return a - delta;
    };

    // (Offsets within a row or an activation buffer stay below 2^24 -- K is at
    // most 32768 and M at most 64 -- so they use the full-rate 24-bit
    // multiply.)
    // One step's global data in registers between load and LDS store.  Every
    // load is issued unconditionally with its address clamped into the
    // buffers (rows past N re-read row N-1, units past K re-read the last
    // one or the row's last 16 bytes, activation rows past M re-read row
    // M-1; none of those reach a stored output): a load behind a branch makes
    // the compiler drain all outstanding loads.
    struct Regs {
        u32x4 wc[WPT];
        u32x4 ac[APT];
        uint32_t dh[SPT];
        int32_t sv[SPT];
    };
    // rowp: the start of the chunk's row (row c / NCH of the workgroup)
    auto chunk_ptr = [&](int st, int c, int& lds_off, const uint8_t* rowp) {
        const int row = c / NCH, k = c - row * NCH;
        if (U::ALIGNED) {
            const int unit = min(G * st + k / 9, nunits - 1);
            lds_off = row * GM::WSTRIDE + 16 * k;
            return rowp + __umul24((unsigned)U::UB, (unsigned)unit) + 16 * (k % 9);
        }
        int delta;
        const uint8_t* a0 = span_base(rowp, st, delta);
        const uint8_t* p = a0 + 16 * k;
        const uint8_t* last = rowp + row_bytes - 16;
        if (p > last) p = last;
        lds_off = row * GM::WSTRIDE + GM::FRONT + (int)(p - a0);
        return p;
    };
    // the rows of this thread's weight chunk slots, the same in every step
    const uint8_t* wrow[WPT];
#pragma unroll
    for (int k = 0; k < WPT; k++)
        wrow[k] = w + (int64_t)min(row0 + min(tid + NT * k, WCH - 1) / NCH, N - 1) * row_bytes;
    auto load_step = [&](int st, Regs& r) {
#pragma unroll
        for (int k = 0; k < WPT; k++) {
            int lo;
            r.wc[k] = ld16(chunk_ptr(st, min(tid + NT * k, WCH - 1), lo, wrow[k]));
        }
#pragma unroll
        for (int k = 0; k < APT; k++) {
            const int c = min(tid + NT * k, ACH - 1);
            const int g = c / (MA * 16), rem = c - g * (MA * 16);
            const int m = min(rem >> 4, M - 1), cc = rem & 15;
            const int u = min(G * st + g, nunits - 1);
            r.ac[k] = *reinterpret_cast<const u32x4*>(q + __umul24((unsigned)m, (unsigned)Kp) + 256 * u + 16 * cc);
        }
#pragma unroll
        for (int k = 0; k < SPT; k++) {
            const int c = min(tid + NT * k, SCH - 1);
            const int g = c / (8 * MA), rem = c - g * (8 * MA);
            const int j = rem / MA, m = min(rem - j * MA, M - 1);
            const int u = min(G * st + g, nunits - 1);
            const int64_t b = __umul24((unsigned)m, (unsigned)nb) + 8 * u + j;
            r.dh[k] = d[b];
            r.sv[k] = s[b];
        }
    };
    auto store_step = [&](const Regs& r, int buf, int st) {
        uint8_t* base = smem + buf * GM::BUF;
#pragma unroll
        for (int k = 0; k < WPT; k++) {
            const int c = tid + NT * k;
            if (c < WCH) {
                int lo;
                (void)chunk_ptr(st, c, lo, wrow[k]);
                *reinterpret_cast<u32x4*>(base + lo) = r.wc[k];
            }
        }
        uint8_t* act = base + GM::WBYTES;
#pragma unroll
        for (int k = 0; k < APT; k++) {
            const int c = tid + NT * k;
            if (c < ACH) {
                const int g = c / (MA * 16), rem = c - g * (MA * 16);
                *reinterpret_cast<u32x4*>(act + g * GM::ASTAGE + (rem >> 4) * GM::ASTRIDE +
                                          16 * (rem & 15)) = r.ac[k];
                if (U::S16) {
                    // sum of these 16 codes (the 16-group rem & 15 of row rem >> 4)
                    int t = dot4(r.ac[k].x, 0x01010101u, 0);
                    t = dot4(r.ac[k].y, 0x01010101u, t);
                    t = dot4(r.ac[k].z, 0x01010101u, t);
                    t = dot4(r.ac[k].w, 0x01010101u, t);
                    int* s16 = reinterpret_cast<int*>(act + g * GM::ASTAGE + GM::ACODES + GM::ASCALE);
                    s16[(rem & 15) * MP + (rem >> 4)] = t;
                }
            }
        }
#pragma unroll
        for (int k = 0; k < SPT; k++) {
            const int c = tid + NT * k;
            if (c < SCH) {
                const int g = c / (8 * MA), rem = c - g * (8 * MA);   // rem = j * MA + m
                const int j = rem / MA, i = j * MP + (rem - j * MA);  // [block][row] slot
                float* dx = reinterpret_cast<float*>(act + g * GM::ASTAGE + GM::ACODES);
                const float f = h2f(r.dh[k]);
                dx[i] = f;
                dx[8 * MP + i] = f * (float)r.sv[k];
            }
        }
    };

    // one accumulator set per unit of a step (G independent chains), or a
    // single set, with the block order pinned, where MT is large and
    // registers are short (Q6_K and Q4_0 need more registers per block)
    constexpr bool BIG = FMT == QGEMV_FMT_Q4_K ? TPW >= 3 : TPW >= 2;
    constexpr int AG = (BIG || KP > 1) ? 1 : G;
    f32x4 acc[AG][TPW], acc2[AG][TPW];
#pragma unroll
    for (int g = 0; g < AG; g++)
#pragma unroll
        for (int t = 0; t < TPW; t++) {
            acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc2[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    const i32x4 zero = {0, 0, 0, 0};
    constexpr int ND = FMT == QGEMV_FMT_Q6_K ? 2 : 1;   // MFMAs (16-groups) per 32-block

    // Unit g of the step in LDS buffer buf, for part P of the 32-blocks (P is
    // the wave's part as a compile-time constant, so field offsets within
    // the unit are constants too).  With PIN set (large MT) empty volatile
    // asm statements make the MFMAs of block jj+1 go out before the scaling
    // of jj and keep every other block in order; without them the compiler
    // issues all the MFMAs first and holds all their results in registers.
    // A unit past the end of K (the tail of the last step) holds stale bytes;
    // its scales are taken as zero, so it adds exact zeros (Q4_0 does the
    // same per block for the blocks of a partial last unit).
    auto compute_sb = [&](auto Pc, auto GAc, int g, int buf, int st, bool valid) {
        constexpr int P = decltype(Pc)::value;
        constexpr int ga = decltype(GAc)::value;   // accumulator set
        // (the dots mode drops the scheduling pins: its stores change the
        // register allocation the pins were placed for; the integer tiles
        // do not depend on the schedule)
        constexpr bool PIN = BIG && !DOTS;
        int delta = 0;
        if (!U::ALIGNED) (void)span_base(my_row, st, delta);
        const int ow = buf * GM::BUF + (16 * rt + nl) * GM::WSTRIDE + GM::FRONT + delta + U::UB * g;
        const int oa = buf * GM::BUF + GM::WBYTES + g * GM::ASTAGE;
        const int blk0 = 8 * (G * st + g);        // first 32-block of the unit
        const float* dxs = reinterpret_cast<const float*>(smem + oa + GM::ACODES + 4 * 8 * MP);

        // format fields of this lane's row
        float fd = 0.0f, fdm = 0.0f;
        uint32_t slo = 0, shi = 0, mlo = 0, mhi = 0;
        if constexpr (FMT == QGEMV_FMT_Q4_K) {
            const u32x4 hdr = *reinterpret_cast<const u32x4*>(smem + ow);
            fd = valid ? h2f(hdr.x & 0xFFFFu) : 0.0f;
            fdm = valid ? h2f(hdr.x >> 16) : 0.0f;
            // 6-bit scales of sub-blocks 0..3 (bytes of hdr.y) and 4..7 (low
            // nibbles of hdr.w, high bits from the top of hdr.y); the mins:
            // bytes of hdr.z, or high nibbles of hdr.w with bits from hdr.z
            slo = hdr.y & 0x3F3F3F3Fu;
            shi = (hdr.w & LO4) | ((hdr.y >> 2) & 0x30303030u);
            mlo = hdr.z & 0x3F3F3F3Fu;
            mhi = ((hdr.w >> 4) & LO4) | ((hdr.z >> 2) & 0x30303030u);
        } else if constexpr (FMT == QGEMV_FMT_Q6_K) {
            // (the scale's bits masked rather than the read skipped: a
            // branch around an LDS read waits for it on the spot)
            fd = h2f(lds2(smem, ow + 208) & (valid ? 0xFFFFu : 0u));
        }
        // Q4_0: the scale of block j of the unit (zero past the row's blocks)
        auto q40_scale = [&](int j) {
            return h2f(lds2(smem, ow + 18 * j) & (blk0 + j < nbw ? 0xFFFFu : 0u));
        };

        auto mfma_block = [&](int jj, i32x4 (&D)[ND][TPW]) {
            const int j = P * BPW + jj;
            int o2 = oa + 32 * j;
            long B[ND];
            if constexpr (FMT == QGEMV_FMT_Q4_K) {
                int o = ow + 16 + 32 * (j >> 1) + 8 * kp;
                if (PIN) asm volatile("" : "+v"(o), "+s"(o2));
                const u32x2 v = *reinterpret_cast<const u32x2*>(smem + o);
                const int sh = 4 * (j & 1);
                B[0] = (long)(((uint64_t)((v.y >> sh) & LO4) << 32) | ((v.x >> sh) & LO4));
            } else if constexpr (FMT == QGEMV_FMT_Q4_0) {
                // block j: element i < 16 = low nibble of byte i, i + 16 = high
                int o = ow + 18 * j + 2 + 8 * (kp & 1);
                if (PIN) asm volatile("" : "+v"(o), "+s"(o2));
                const u32x2 v = lds8_a2(smem, o);
                const int sh = 4 * (kp >> 1);
                B[0] = (long)(((uint64_t)((v.y >> sh) & LO4) << 32) | ((v.x >> sh) & LO4));
            } else {
                // block j = 4h + t: element l of it = low (t < 2) or high
                // (t >= 2) nibble of ql[64h + 32(t&1) + l], plus bits 2t..2t+1
                // of qh[32h + l] as bits 4..5
                const int h = j >> 2, t = j & 3;
                int o = ow + 64 * h + 32 * (t & 1) + 8 * kp;
                int oh = ow + 128 + 32 * h + 8 * kp;
                if (PIN) asm volatile("" : "+v"(o), "+v"(oh), "+s"(o2));
                const u32x2 ql = lds8_a2(smem, o);
                const u32x2 qh = lds8_a2(smem, oh);
                const int s1 = 4 * (t >> 1), s2 = 2 * t;
                const uint32_t c0 = ((ql.x >> s1) & LO4) | (((qh.x >> s2) & 0x03030303u) << 4);
                const uint32_t c1 = ((ql.y >> s1) & LO4) | (((qh.y >> s2) & 0x03030303u) << 4);
                const long Bc = (long)(((uint64_t)c1 << 32) | c0);
                // 16-group 2j is K lanes kp < 2, group 2j+1 kp >= 2 (with one
                // activation tile the A operand is split instead, below)
                B[0] = ZA || kp < 2 ? Bc : 0;
                B[1] = ZA || kp >= 2 ? Bc : 0;
            }
            if constexpr (FMT == QGEMV_FMT_Q6_K && ZA) {
                // lanes kp < 2 supply their codes to the first MFMA and zeros
                // (from the zero block) to the second, lanes kp >= 2 the
                // other way round
                const int oc = o2 + (16 * t0 + nl) * GM::ASTRIDE + 8 * kp;
                const long A0 = *reinterpret_cast<const long*>(smem + (kp < 2 ? oc : ZOFF + 8 * kp));
                const long A1 = *reinterpret_cast<const long*>(smem + (kp < 2 ? ZOFF + 8 * kp : oc));
                D[0][0] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A0, B[0], zero, 0, 0, 0);
                D[1][0] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A1, B[1], zero, 0, 0, 0);
            } else {
#pragma unroll
                for (int t = 0; t < TPW; t++) {
                    const long A = *reinterpret_cast<const long*>(
                        smem + o2 + (16 * (t0 + t) + nl) * GM::ASTRIDE + 8 * kp);
#pragma unroll
                    for (int e = 0; e < ND; e++)
                        D[e][t] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B[e], zero, 0, 0, 0);
                }
            }
            if constexpr (DOTS) {
                // outputs of lane l: activation rows 16t + 4(l/16) + i of weight row n
                const int blk = blk0 + j;
                const bool okb = valid && n < N && (FMT != QGEMV_FMT_Q4_0 || blk < nbw);
                const int ndb = FMT == QGEMV_FMT_Q6_K ? 2 * nb : (FMT == QGEMV_FMT_Q4_0 ? nbw : nb);
#pragma unroll
                for (int t = 0; t < TPW; t++)
#pragma unroll
                    for (int e = 0; e < ND; e++)
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            const int m = 16 * (t0 + t) + 4 * kp + i;
                            const int col = FMT == QGEMV_FMT_Q6_K ? 2 * blk + e : blk;
                            if (okb && m < M)
                                dots[((int64_t)m * N + n) * ndb + col] = D[e][t][i];
                        }
            }
        };
        auto scale_block = [&](int jj, const i32x4 (&D)[ND][TPW]) {
            const int j = P * BPW + jj;
            float ws0, ws1 = 0.0f;
            if constexpr (FMT == QGEMV_FMT_Q4_K) {
                ws0 = fd * (float)(((j >= 4 ? shi : slo) >> (8 * (j & 3))) & 0xFFu);
            } else if constexpr (FMT == QGEMV_FMT_Q4_0) {
                ws0 = q40_scale(j);
            } else {
                const uint32_t sc = lds2(smem, ow + 192 + 2 * j);   // int8 scales of 2j, 2j+1
                ws0 = fd * (float)sbyte(sc, 0);
                ws1 = fd * (float)sbyte(sc, 1);
            }
            int o = oa + GM::ACODES + 4 * j * MP;
            if (PIN) asm volatile("" : "+s"(o));
#pragma unroll
            for (int t = 0; t < TPW; t++) {
                const f32x4 x4 =
                    *reinterpret_cast<const f32x4*>(smem + o + 4 * (16 * (t0 + t) + 4 * kp));
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    if constexpr (ND == 1) {
                        acc[ga][t][i] = fmaf((float)D[0][t][i], ws0 * x4[i], acc[ga][t][i]);
                    } else {
                        const float v = fmaf((float)D[1][t][i], ws1, (float)D[0][t][i] * ws0);
                        acc[ga][t][i] = fmaf(v, x4[i], acc[ga][t][i]);
                    }
                }
            }
            if (PIN) {
#pragma unroll
                for (int t = 0; t < TPW; t++) asm volatile("" : "+v"(acc[ga][t]));
            }
        };
        // Two-block tiles (at most 8 activation rows): one
        // v_mfma_i32_16x16x64_i8 per pair of 32-blocks (jp, jp + 1).  Tile
        // rows 0-7 are activation rows 0-7 against block jp (K lanes 0-31, the
        // quarters kp < 2; zeros in K lanes 32-63) and rows 8-15 the same
        // activation rows against block jp + 1 (K lanes 32-63), so every
        // output is one exact block dot and no tile row is padding.  Lane
        // (nl, kp) holds rows 4*kp + i: block jp + (kp >= 2) of activation row
        // 4*(kp & 1) + i; the two halves of a row meet at the end.
        auto mfma_pair = [&](int pi, i32x4 (&E)[ND]) {
            const int jp = P * BPW + 2 * pi;              // even block of the pair
            const int jb = jp + (kp >> 1);                // this lane's block
            // weights: 16 codes of block jb for K lanes 16*kp .. 16*kp + 15
            // (elements 16*(kp & 1) .. of the block)
            i32x4 B;
            if constexpr (FMT == QGEMV_FMT_Q4_K) {
                // bytes 32*(jp/2) + 16*(kp&1) .. +15 of the unit's codes: low
                // nibbles are block jp, high nibbles block jp + 1
                const u32x4 v = *reinterpret_cast<const u32x4*>(smem + ow + 16 + 16 * jp + 16 * (kp & 1));
                const int sh = kp < 2 ? 0 : 4;
                B = i32x4{(int)((v.x >> sh) & LO4), (int)((v.y >> sh) & LO4),
                          (int)((v.z >> sh) & LO4), (int)((v.w >> sh) & LO4)};
            } else if constexpr (FMT == QGEMV_FMT_Q4_0) {
                // block jb's 16 bytes: elements 0-15 are the low nibbles,
                // 16-31 the high nibbles
                const u32x4 v = lds16_a2(smem, ow + 18 * jb + 2);
                const int sh = 4 * (kp & 1);
                B = i32x4{(int)((v.x >> sh) & LO4), (int)((v.y >> sh) & LO4),
                          (int)((v.z >> sh) & LO4), (int)((v.w >> sh) & LO4)};
            } else {
                // block jb = 4h + t: element l = low (t < 2) or high nibble of
                // ql[64h + 32(t&1) + l], plus bits 2t..2t+1 of qh[32h + l]
                const int h = jb >> 2, tt = jb & 3;
                const u32x4 ql = lds16_a2(smem, ow + 64 * h + 32 * (tt & 1) + 16 * (kp & 1));
                const u32x4 qh = lds16_a2(smem, ow + 128 + 32 * h + 16 * (kp & 1));
                const int s1 = 4 * (tt >> 1), s2 = 2 * tt;
                B = i32x4{(int)(((ql.x >> s1) & LO4) | (((qh.x >> s2) & 0x03030303u) << 4)),
                          (int)(((ql.y >> s1) & LO4) | (((qh.y >> s2) & 0x03030303u) << 4)),
                          (int)(((ql.z >> s1) & LO4) | (((qh.z >> s2) & 0x03030303u) << 4)),
                          (int)(((ql.w >> s1) & LO4) | (((qh.w >> s2) & 0x03030303u) << 4))};
            }
            // A operand: lane (nl, kp) carries activation row nl & 7 of block
            // jb where tile row nl belongs to that block (mine), else zeros,
            // read from the zero block (same offsets within it)
            const int off = 32 * jb + 16 * (kp & 1);
            const bool mine = (nl < 8) == (kp < 2);
            auto a_load = [&](bool real) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(
                    smem + (real ? oa + (nl & 7) * GM::ASTRIDE : ZOFF) + off);
                return i32x4{(int)a.x, (int)a.y, (int)a.z, (int)a.w};
            };
            if constexpr (ND == 1) {
                E[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_load(mine), B, zero, 0, 0, 0);
            } else {
                // Q6_K: a lane's K values are one 16-group (2*jb + (kp & 1));
                // the first MFMA takes the first group of each block (lanes
                // with kp even supply codes, the others zeros), the second
                // the other
                const bool g1 = (kp & 1) != 0;
                E[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_load(mine && !g1), B, zero, 0, 0, 0);
                E[1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_load(mine && g1), B, zero, 0, 0, 0);
            }
            if constexpr (DOTS) {
                const int blk = blk0 + jb;
                const bool okb = valid && n < N && (FMT != QGEMV_FMT_Q4_0 || blk < nbw);
                const int ndb = FMT == QGEMV_FMT_Q6_K ? 2 * nb : (FMT == QGEMV_FMT_Q4_0 ? nbw : nb);
#pragma unroll
                for (int e = 0; e < ND; e++)
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const int m = 4 * (kp & 1) + i;
                        const int col = FMT == QGEMV_FMT_Q6_K ? 2 * blk + e : blk;
                        if (okb && m < M) dots[((int64_t)m * N + n) * ndb + col] = E[e][i];
                    }
            }
        };
        auto scale_pair = [&](int pi, const i32x4 (&E)[ND]) {
            const int jp = P * BPW + 2 * pi;
            const int jb = jp + (kp >> 1);
            const f32x4 x4 = *reinterpret_cast<const f32x4*>(
                smem + oa + GM::ACODES + 4 * (jb * MP + 4 * (kp & 1)));
            if constexpr (ND == 1) {
                float ws;
                if constexpr (FMT == QGEMV_FMT_Q4_K)
                    ws = fd * (float)(((jb >= 4 ? shi : slo) >> (8 * (jb & 3))) & 0xFFu);
                else
                    ws = q40_scale(jb);
#pragma unroll
                for (int i = 0; i < 4; i++) acc[ga][0][i] = fmaf((float)E[0][i], ws * x4[i], acc[ga][0][i]);
            } else {
                const uint32_t sc = lds2(smem, ow + 192 + 2 * jb);   // int8 scales of 2jb, 2jb+1
                const float ws0 = fd * (float)sbyte(sc, 0), ws1 = fd * (float)sbyte(sc, 1);
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const float v = fmaf((float)E[1][i], ws1, (float)E[0][i] * ws0);
                    acc[ga][0][i] = fmaf(v, x4[i], acc[ga][0][i]);
                }
            }
        };
        if constexpr (TWO) {
            i32x4 E2[2][ND];
            mfma_pair(0, E2[0]);
#pragma unroll
            for (int pi = 1; pi < BPW / 2; pi++) {
                mfma_pair(pi, E2[pi & 1]);
                scale_pair(pi - 1, E2[(pi - 1) & 1]);
            }
            scale_pair(BPW / 2 - 1, E2[(BPW / 2 - 1) & 1]);
        } else {
            i32x4 D2[2][ND][TPW];
            mfma_block(0, D2[0]);
#pragma unroll
            for (int jj = 1; jj < BPW; jj++) {
                mfma_block(jj, D2[jj & 1]);
                scale_block(jj - 1, D2[(jj - 1) & 1]);
            }
            scale_block(BPW - 1, D2[(BPW - 1) & 1]);
        }

        // the second products: K lane kp of an fp32 MFMA carries one block
        // (Q4_K, Q4_0: block 4*kk + kp of the unit, lanes whose block belongs
        // to another wave contribute zero) or one 16-group (Q6_K)
        if constexpr (FMT == QGEMV_FMT_Q6_K) {
            const int* s16 = reinterpret_cast<const int*>(smem + oa + GM::ACODES + GM::ASCALE);
            const float* dx = reinterpret_cast<const float*>(smem + oa + GM::ACODES);
#pragma unroll
            for (int kk = 0; kk < BPW / 2; kk++) {
                const int gi = 2 * P * BPW + 4 * kk + kp;   // this lane's 16-group
                const uint32_t sc = lds2(smem, ow + 192 + (gi & ~1));
                const float b = 32.0f * fd * (float)sbyte(sc, gi & 1);
#pragma unroll
                for (int t = 0; t < TPW; t++) {
                    const int m = 16 * (t0 + t) + nl;
                    // (two-block tiles stage activation rows 0-7 only)
                    const float a = TWO && nl >= 8 ? 0.0f : dx[(gi >> 1) * MP + m] * (float)s16[gi * MP + m];
                    acc2[ga][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc2[ga][t], 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < (BPW == 8 ? 2 : 1); kk++) {
                constexpr int JB = BPW == 8 ? 0 : (P * BPW) & ~3;   // first block of the group
                const int jg = BPW == 8 ? 4 * kk : JB;
                const bool mine = BPW >= 4 || (kp >> 1) == (P & 1);
                float b;
                if constexpr (FMT == QGEMV_FMT_Q4_K) {
                    const uint32_t mb = jg >= 4 ? mhi : mlo;
                    b = mine ? fdm * (float)bfe(mb, 8 * kp, 8) : 0.0f;
                } else {
                    b = mine ? 8.0f * q40_scale(jg + kp) : 0.0f;
                }
#pragma unroll
                for (int t = 0; t < TPW; t++) {
                    // (two-block tiles stage activation rows 0-7 only)
                    const float a = TWO && nl >= 8 ? 0.0f : dxs[(jg + kp) * MP + 16 * (t0 + t) + nl];
                    acc2[ga][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc2[ga][t], 0, 0, 0);
                }
            }
        }
    };
    auto compute_part = [&](auto Pc, int buf, int st) {
        if (KP == 1) {
            compute_sb(Pc, std::integral_constant<int, 0>{}, 0, buf, st, true);
            if (G > 1)
                compute_sb(Pc, std::integral_constant<int, (AG > 1 ? 1 : 0)>{}, 1, buf, st,
                           G * st + 1 < nunits);
        } else {
            for (int g = kq; g < G; g += KP)
                compute_sb(Pc, std::integral_constant<int, 0>{}, g, buf, st, G * st + g < nunits);
        }
    };
    auto compute_step = [&](int buf, int st) {
        if (KS == 1) {
            compute_part(std::integral_constant<int, 0>{}, buf, st);
        } else if (KS == 2) {
            if (ks == 0) compute_part(std::integral_constant<int, 0>{}, buf, st);
            else compute_part(std::integral_constant<int, 1>{}, buf, st);
        } else {
            switch (ks) {
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
    // buffer.  It starts at st = -R with nothing loaded.  With R > 1 every
    // step issues the same loads (the last ones again at the end), so the
    // compiler's wait counts stay exact; with R = 1 the store waits for all
    // of the step's loads anyway, and the last step issues none (a load
    // left in flight there would hold up the epilogue by a full latency).
    Regs rg[R];
    for (int base = -R; base < nsteps; base += R) {
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int st = base + r;
            if (R > 1 || st + R < nsteps) load_step(min(st + R, nsteps - 1), rg[r]);
            __builtin_amdgcn_sched_barrier(0);
            if (st >= 0 && st < nsteps) compute_step(st & 1, st);
            if (st + 1 >= 0 && st + 1 < nsteps) store_step(rg[(r + 1) % R], (st + 1) & 1, st + 1);
            __syncthreads();
        }
    }

    // partial sums of parts 1 .. KS-1 go through LDS (free after the last
    // step's barrier); part 0 adds them in part order and stores
    float* pbuf = reinterpret_cast<float*>(smem);
    auto partial = [&](int t, int i) {
        if constexpr (TWO) {
            // lanes kp < 2 hold the even blocks of rows 4*kp + i, lanes 32
            // above them the odd blocks of the same rows
            float a = acc[0][t][i], m2 = acc2[0][t][i];
#pragma unroll
            for (int g = 1; g < AG; g++) {
                a += acc[g][t][i];
                m2 += acc2[g][t][i];
            }
            return (a + __shfl_xor(a, 32)) - m2;
        }
        float v = acc[0][t][i] - acc2[0][t][i];
#pragma unroll
        for (int g = 1; g < AG; g++) v += acc[g][t][i] - acc2[g][t][i];
        return v;
    };
    auto pidx = [&](int p, int t, int i) {   // t: this wave's tile index 0 .. TPW-1
        return (((p - 1) * RT + rt) * MT * 4 + 4 * (t0 + t) + i) * 64 + lane;
    };
    // (formed by every lane of the wave: the two-block halves meet across lanes)
    float pv[TPW][4];
#pragma unroll
    for (int t = 0; t < TPW; t++)
#pragma unroll
        for (int i = 0; i < 4; i++) pv[t][i] = partial(t, i);
    if (NPART > 1 && part > 0) {
#pragma unroll
        for (int t = 0; t < TPW; t++)
#pragma unroll
            for (int i = 0; i < 4; i++) pbuf[pidx(part, t, i)] = pv[t][i];
    }
    if (NPART > 1) __syncthreads();
    if (part == 0 && n < N) {
#pragma unroll
        for (int t = 0; t < TPW; t++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                float v = pv[t][i];
#pragma unroll
                for (int p = 1; p < NPART; p++) v += pbuf[pidx(p, t, i)];
                const int m = 16 * (t0 + t) + 4 * kp + i;
                if (m < M) y[(int64_t)m * N + n] = v;
            }
    }
}

// RT: weight tiles per workgroup (the activation staged by a workgroup is
// shared by 16*RT weight rows); KS, KP: waves sharing a tile's 32-blocks and
// units; G: units per step; R: steps of global loads in flight.
template <int FMT, int MT, int RT, int KS, int KP, int MS, int G, int R, bool DOTS,
          bool TWO = false>
static hipError_t launch_mfma_cfg(const void* w, int64_t N, int64_t K, int64_t M,
                                  const int8_t* q, const uint16_t* d, const int32_t* s, float* y,
                                  int32_t* dots, hipStream_t st) {
    const int Kp = (int)((K + 255) / 256 * 256);
    const int64_t grid = (N + 16 * RT - 1) / (16 * RT);
    const int64_t mgroups = (M + 16 * MT - 1) / (16 * MT);   // activation row groups
    launch_kernel((k_small_m_mfma<FMT, MT, RT, KS, KP, MS, G, R, DOTS, TWO>),
                  dim3((unsigned)grid, (unsigned)mgroups),
                  dim3(64 * RT * KS * KP * MS), 0, st, (const uint8_t*)w, (int)N, (int)K,
                  Kp, (int)M, q, d, s, y, dots);
    return hipGetLastError();
}

// Matrices with fewer 16-row tiles than this also split K between waves.
constexpr int64_t kMfmaWideTiles = 512;

// Row m of a product depends only on activation row m and on the bucket of
// M (1-8: two-block tiles; 9-16, 17-32, 33-48, 49-64 rows) and the shape,
// which fix the configuration and so the fp32 summation order.
// Wide Q4_K matrices at M = 33-64: 32 activation rows per workgroup (a
// second grid dimension takes the rest) against 64 weight rows, whole units
// per wave, one step of loads in flight -- 8 waves of ~118 VGPRs, so two
// workgroups share a unit, where 64 activation rows per workgroup (~194
// VGPRs) left two waves per SIMD.  Measured against the 64-by-64 workgroups
// (same process): 27.1 against 33.2 us at M = 64 on 14336 x 4096, 51.3
// against 64.5 us on 28672 x 4096, 217 against 251 us on 128256 x 4096; 26.1
// against 27.9 us at M = 48 and 26.2 against 27.5 us at M = 40.
template <bool DOTS>
static hipError_t launch_q4k_wide_split(const void* w, int64_t N, int64_t K, int64_t M,
                                        const int8_t* q, const uint16_t* d, const int32_t* s,
                                        float* y, int32_t* dots, hipStream_t st) {
    return launch_mfma_cfg<QGEMV_FMT_Q4_K, 2, 4, 1, 2, 1, 2, 1, DOTS>(w, N, K, M, q, d, s, y,
                                                                       dots, st);
}

template <int FMT, bool DOTS = false>
static hipError_t launch_mfma(const void* w, int64_t N, int64_t K, int64_t M, const int8_t* q,
                              const uint16_t* d, const int32_t* s, float* y, hipStream_t st,
                              int32_t* dots = nullptr) {
    const int mt = (int)((M + 15) / 16);
    const bool wide = (N + 15) / 16 >= kMfmaWideTiles;
    // <FMT, MT, RT, KS, KP, MS, G, R>.  Wide matrices: 32 (MT = 1) or 64
    // weight rows per workgroup share the staged activation and each wave
    // takes every activation tile (splitting the tiles there costs more
    // activation traffic than it gains; Q6_K's larger units leave LDS for 2
    // row tiles from MT = 3).  Narrow matrices also split K between waves (at
    // MT = 1 the 4 units of a step and the two halves of each unit's
    // 32-blocks over 8 waves: 6% faster on Q6_K 4096x14336 than 8 units over
    // 8 waves) and, from MT = 2, give each wave one activation tile (MS = MT),
    // so a wave needs the registers of MT = 1 and the chip gets MT times the
    // waves.  The per-format choices below were each measured against the
    // alternative in one process; a bucket of M and a shape fix the
    // configuration, so the summation order stays fixed per row.
    constexpr int RT34 = FMT == QGEMV_FMT_Q6_K ? 2 : 4;
    if (wide) {
        switch (mt) {
        case 1:
            // Every format: each wave takes whole units (measured faster than
            // halving each unit's 32-blocks over 2 more waves, same process:
            // Q4_K 14336 x 4096 at M = 16 14.1 against 14.9 us, Q6_K 12288 x
            // 4096 at M = 8 23.2 against 24.5 us, Q4_0 14336 x 4096 at M = 8
            // 18.2 against 18.9 us).  Q4_K: 4 units per step on 4 waves (8
            // per workgroup of 32 rows), one step of loads in flight: 11.0
            // against 12.9 us at M = 8 and 13.4 against 15.2 us at M = 16 on
            // 14336 x 4096, 20.3 against 21.7 us at M = 8 on 28672 x 4096;
            // Q6_K and Q4_0 lose so (Q6_K 12288 x 4096 M = 8 24.7 against
            // 22.7 us, Q4_0 14336 x 4096 M = 8 17.6 against 16.2 us).  Q4_0
            // at M <= 8: the 2 units of a step on 2 waves with one step in
            // flight, 15.3 against 16.2 us (two in flight stay faster for
            // Q6_K: 153.7 against 156.8 us on 128256 x 4096).  At most 8
            // activation rows: two-block tiles, two 32-blocks per i8 MFMA with
            // no padding rows (M = 8 against M = 9 with the same split: Q4_K
            // 12.3 against 13.9 us, Q6_K 12288 x 4096 22.1 against 23.1 us,
            // Q4_0 15.8 against 18.2 us; Q4_K 28672 x 4096 19.6 against
            // 24.9 us)
            if constexpr (FMT == QGEMV_FMT_Q4_K) {
                if (M <= 8)
                    return launch_mfma_cfg<FMT, 1, 2, 1, 4, 1, 4, 1, DOTS, true>(w, N, K, M, q, d, s, y, dots, st);
                return launch_mfma_cfg<FMT, 1, 2, 1, 4, 1, 4, 1, DOTS>(w, N, K, M, q, d, s, y, dots, st);
            } else if constexpr (FMT == QGEMV_FMT_Q4_0) {
                if (M <= 8)
                    return launch_mfma_cfg<FMT, 1, 2, 1, 2, 1, 2, 1, DOTS, true>(w, N, K, M, q, d, s, y, dots, st);
            } else {
                if (M <= 8)
                    return launch_mfma_cfg<FMT, 1, 2, 1, 2, 1, 2, 2, DOTS, true>(w, N, K, M, q, d, s, y, dots, st);
            }
            return launch_mfma_cfg<FMT, 1, 2, 1, 2, 1, 2, 2, DOTS>(w, N, K, M, q, d, s, y, dots, st);
        case 2:
            // Q4_K: the units of a step on 2 waves each: 19.7 against 21.8 us
            // at M = 24 on 14336 x 4096 (same process), and with one step of
            // loads in flight 17.6 against 19.0 us; Q6_K runs slower so.
            // Q4_0: whole units per wave, the 2 units of a step on 2 waves:
            // 24.6 against 25.2 us at M = 24 (same process)
            if constexpr (FMT == QGEMV_FMT_Q4_K)
                return launch_mfma_cfg<FMT, 2, 4, 2, 2, 1, 2, 1, DOTS>(w, N, K, M, q, d, s, y, dots, st);
            else if constexpr (FMT == QGEMV_FMT_Q4_0)
                return launch_mfma_cfg<FMT, 2, 4, 1, 2, 1, 2, 2, DOTS>(w, N, K, M, q, d, s, y, dots, st);
            else
                return launch_mfma_cfg<FMT, 2, 4, 2, 1, 1, 2, 2, DOTS>(w, N, K, M, q, d, s, y, dots, st);
        case 3:
            // Q4_0: each wave takes whole units (all 8 32-blocks), the 2
            // units of a step on 2 waves: 32.2 against 32.9 us at M = 40 on
            // 14336 x 4096 (same process)
            if constexpr (FMT == QGEMV_FMT_Q6_K)
                return launch_mfma_cfg<FMT, 3, RT34, 2, 2, 1, 2, 2, DOTS>(w, N, K, M, q, d, s, y, dots, st);
            else if constexpr (FMT == QGEMV_FMT_Q4_0)
                return launch_mfma_cfg<FMT, 3, RT34, 1, 2, 1, 2, 2, DOTS>(w, N, K, M, q, d, s, y, dots, st);
            else
                return launch_q4k_wide_split<DOTS>(w, N, K, M, q, d, s, y, dots, st);
        default:
            // Q6_K: the units of a step on 2 waves each: 71 against 119 us at
            // M = 64 on 12288 x 4096 (same process).  Q4_0: 32 activation
            // rows per workgroup (a second grid dimension takes the rest),
            // 128 weight rows, whole units per wave and one step of loads in
            // flight: 35.2 against 38.8 us at M = 64 on 14336 x 4096 with 64
            // rows by 64
            if constexpr (FMT == QGEMV_FMT_Q6_K)
                return launch_mfma_cfg<FMT, 4, RT34, 2, 2, 1, 2, 2, DOTS>(w, N, K, M, q, d, s, y, dots, st);
            else if constexpr (FMT == QGEMV_FMT_Q4_0)
                return launch_mfma_cfg<FMT, 2, 8, 1, 2, 1, 2, 1, DOTS>(w, N, K, M, q, d, s, y, dots, st);
            else
                return launch_q4k_wide_split<DOTS>(w, N, K, M, q, d, s, y, dots, st);
        }
    }
    switch (mt) {
    case 1:
        // at most 8 rows: two-block tiles (M = 8 against M = 9 on 4096 x
        // 14336: Q4_K 13.4 against 15.7 us, Q6_K 22.8 against 25.1 us, Q4_0
        // 17.1 against 20.5 us), and 8 units per step over 8 waves (each
        // unit's 32-blocks halved over 2 of 16 waves) with one step of loads
        // in flight against 4 units and two steps: Q4_0 14.6 against 17.3
        // us, Q6_K 20.9 against 22.7 us, Q4_K 13.6 against 13.8 us.  At 9-16
        // rows the same for Q4_0 (19.1 against 21.1 us) and Q6_K (22.8
        // against 26.4 us); Q4_K stays on 4 units (17.0 against 18.4 us).
        if (M <= 8)
            return launch_mfma_cfg<FMT, 1, 1, 2, 8, 1, 8, 1, DOTS, true>(w, N, K, M, q, d, s, y, dots, st);
        if constexpr (FMT != QGEMV_FMT_Q4_K)
            return launch_mfma_cfg<FMT, 1, 1, 2, 8, 1, 8, 1, DOTS>(w, N, K, M, q, d, s, y, dots, st);
        else
            return launch_mfma_cfg<FMT, 1, 1, 2, 4, 1, 4, 2, DOTS>(w, N, K, M, q, d, s, y, dots, st);
    case 2:
        // Q4_K: each unit's 32-blocks halved over 2 waves: 25.4 against 29.1
        // us at M = 24 on 4096 x 14336 (same process).  Q6_K and Q4_0: 4
        // units per step, each halved over 2 waves, one step of loads in
        // flight: on 4096 x 14336 at M = 24 Q6_K 37.8 against 44.7 us (4
        // whole units per step, two in flight) and Q4_0 28.3 against 33.3 us
        // (the Q4_K split); Q4_K loses so (27.5 against 24.7 us)
        if constexpr (FMT == QGEMV_FMT_Q4_K)
            return launch_mfma_cfg<FMT, 2, 1, 2, 2, 2, 2, 2, DOTS>(w, N, K, M, q, d, s, y, dots, st);
        else
            return launch_mfma_cfg<FMT, 2, 1, 2, 4, 2, 4, 1, DOTS>(w, N, K, M, q, d, s, y, dots, st);
    case 3:
        // the same split for every format: at M = 48 on 4096 x 14336, Q6_K
        // 57 against 73 us, Q4_K 38 against 46 us, Q4_0 48 against 63 us
        return launch_mfma_cfg<FMT, 3, 1, 2, 2, 3, 2, 2, DOTS>(w, N, K, M, q, d, s, y, dots, st);
    default:
        // Q4_K and Q4_0: 32 activation rows per workgroup (a second grid
        // dimension takes the rest) with the M = 17-32 splits, at M = 64 on
        // 4096 x 14336 Q4_K 46.2 against 50.8 us and Q4_0 56.3 against 69.9
        // us (64 rows per workgroup, each wave one tile of 16); Q6_K keeps
        // that (and under AUTO takes the wave-stream kernel)
        if constexpr (FMT == QGEMV_FMT_Q4_K)
            return launch_mfma_cfg<FMT, 2, 1, 2, 2, 2, 2, 2, DOTS>(w, N, K, M, q, d, s, y, dots, st);
        else if constexpr (FMT == QGEMV_FMT_Q4_0)
            return launch_mfma_cfg<FMT, 2, 1, 2, 4, 2, 4, 1, DOTS>(w, N, K, M, q, d, s, y, dots, st);
        else
            return launch_mfma_cfg<FMT, 4, 1, 1, 2, 4, 2, 2, DOTS>(w, N, K, M, q, d, s, y, dots, st);
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
    launch_kernel((k_small_m_dot4<MT, LPR>), dim3((unsigned)gx, (unsigned)gy), dim3(SWG),
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

// AUTO: the MFMA variant from this many rows on (measured crossovers on
// MI355X, same process: wide Q4_K takes 12.9 us at M = 3 through the
// streaming rows and 12.1 us on MFMA's two-block tiles on 14336 x 4096, 20.0
// against 18.8 us on 28672 x 4096; narrow Q4_K 4096 x 14336 12.6 against
// 13.4 us at M = 4; Q6_K 4096 x 14336 16.6 against 22.6 us and Q4_0 14336 x
// 4096 12.9 against 15.6 us at M = 4, while two passes of four rows lose to
// MFMA from M = 5 everywhere).
static int mfma_from_m(int fmt, int64_t N) {
    if (fmt == QGEMV_FMT_Q4_K && (N + 15) / 16 >= kMfmaWideTiles) return 3;
    return 5;
}

static hipError_t launch_dot4_q4k(const void* w, int64_t N, int64_t K, int64_t M,
                                  const int8_t* q, const uint16_t* d, const int32_t* s, float* y,
                                  hipStream_t st) {
    int mt = dot4_tile_rows(K);
    if (M < mt) mt = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8;
    switch (mt) {
    case 8: return launch_dot4_mt<8>(w, N, K, M, q, d, s, y, st);
    case 4: return launch_dot4_mt<4>(w, N, K, M, q, d, s, y, st);
    case 2: return launch_dot4_mt<2>(w, N, K, M, q, d, s, y, st);
    default: return launch_dot4_mt<1>(w, N, K, M, q, d, s, y, st);
    }
}

// The DOT4 variant of the Q6_K and Q4_0 products: the batch-1 GEMV on each
// activation row (row m of the product is by definition that GEMV).
static hipError_t launch_rows_gemv(int fmt, const void* w, int64_t N, int64_t K, int64_t M,
                                   const int8_t* q, const uint16_t* d, const int32_t* s,
                                   float* y, hipStream_t st) {
    const int64_t Kp = (K + 255) / 256 * 256;
    for (int64_t m = 0; m < M; m++) {
        const GemvArgs a{w, N, K, q + m * Kp, d + m * (Kp / 32), s + m * (Kp / 32), y + m * N};
        const hipError_t e = launch_gemv(fmt, a, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Which int8-MFMA kernel takes a product: the wave-stream kernel
// (k_small_m2.hip) where it measured faster than the staged one -- Q6_K from
// M = 17 (4096 x 14336: 48.3 against 82.8 us at M = 64, 42.7 against 57.0 us
// at M = 48, 37.3 against 37.6 us at M = 17; 12288 x 4096: 49.3 against 72.4
// us at M = 64, 36.2 against 57.1 us at M = 48, 31.9 against 34.5 us at M =
// 17) -- the staged kernel elsewhere (Q4_K 14336 x 4096: 13.6 against
// 17.9 us at M = 8, 33.8 against 36.0 us at M = 64; Q4_0: 19.1 against 51.6
// us at M = 8).  A shape and a bucket of M fix the kernel, so the summation
// order of a row stays fixed.
// Which products the register-resident kernel (k_small_m3.hip) takes under
// MFMA and AUTO: Q4_K with 9 to 16 rows on matrices of at least six 16-row
// tiles per compute unit, where it measured faster than the 16-row tiles
// (28672 x 4096 at M = 8: 22.2 against 24.8 us staged; 14336 x 4096: 15.0
// against 13.5 us, so narrower matrices stay with the staged kernel).  Up to
// 8 rows the staged kernel's two-block tiles beat both (19.6 us at M = 8 on
// 28672 x 4096).
static bool use_resident_kernel(int fmt, int64_t N, int64_t K, int64_t M) {
    // (at most 8 rows the staged kernel's two-block tiles are faster there too)
    if (M <= 8 || !small_m3_supported(fmt, K, M)) return false;
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0) {
        (void)hipGetLastError();
        cus = 256;
    }
    return (N + 15) / 16 >= 6 * (int64_t)cus;
}

static bool use_stream_kernel(int fmt, int64_t N, int64_t M) {
    (void)N;
    return fmt == QGEMV_FMT_Q6_K && M >= 17;
}

hipError_t launch_small_m(int fmt, const void* w, int64_t N, int64_t K, int64_t M,
                          const int8_t* q, const uint16_t* d, const int32_t* s, float* y,
                          int variant, hipStream_t st) {
    const bool auto_mfma = variant == QGEMV_VARIANT_AUTO && M >= mfma_from_m(fmt, N);
    if ((variant == QGEMV_VARIANT_MFMA_RESIDENT && small_m3_supported(fmt, K, M)) ||
        ((variant == QGEMV_VARIANT_MFMA || auto_mfma) && use_resident_kernel(fmt, N, K, M)))
        return launch_small_m3(fmt, w, N, K, M, q, d, s, y, st);
    if (variant == QGEMV_VARIANT_MFMA_RESIDENT) variant = QGEMV_VARIANT_MFMA;
    if (variant == QGEMV_VARIANT_MFMA_STREAM ||
        ((variant == QGEMV_VARIANT_MFMA || auto_mfma) && use_stream_kernel(fmt, N, M)))
        return launch_small_m2(fmt, w, N, K, M, q, d, s, y, st);
    const bool mfma =
        variant == QGEMV_VARIANT_MFMA || variant == QGEMV_VARIANT_MFMA_STAGED || auto_mfma;
    if (!mfma) {
        // one row: the batch-1 GEMV; more: up to four rows per pass of the
        // batch-1 streaming kernel, else the GEMV on each row
        if (M == 1) return launch_rows_gemv(fmt, w, N, K, M, q, d, s, y, st);
        const hipError_t e = launch_small_m_rows(fmt, w, N, K, M, q, d, s, y, st);
        if (e != hipErrorNotSupported) return e;
        if (fmt == QGEMV_FMT_Q4_K) return launch_dot4_q4k(w, N, K, M, q, d, s, y, st);
        return launch_rows_gemv(fmt, w, N, K, M, q, d, s, y, st);
    }
    switch (fmt) {
    case QGEMV_FMT_Q4_K: return launch_mfma<QGEMV_FMT_Q4_K>(w, N, K, M, q, d, s, y, st);
    case QGEMV_FMT_Q6_K: return launch_mfma<QGEMV_FMT_Q6_K>(w, N, K, M, q, d, s, y, st);
    default: return launch_mfma<QGEMV_FMT_Q4_0>(w, N, K, M, q, d, s, y, st);
    }
}

// Whether the kernel variant selects for (fmt, N, K, M) has a dots mode (not
// the wave-stream kernel).  Uses the device's compute-unit count where it
// decides (256 without a device).
bool small_m_dots_supported(int fmt, int64_t N, int64_t K, int64_t M, int variant) {
    if (variant == QGEMV_VARIANT_MFMA_STAGED) return true;
    if (variant == QGEMV_VARIANT_MFMA_RESIDENT && small_m3_supported(fmt, K, M)) return true;
    if (variant == QGEMV_VARIANT_MFMA && use_resident_kernel(fmt, N, K, M)) return true;
    return !use_stream_kernel(fmt, N, M);
}

hipError_t launch_small_m_dots(int fmt, const void* w, int64_t N, int64_t K, int64_t M,
                               const int8_t* q, const uint16_t* d, const int32_t* s, float* y,
                               int variant, int32_t* dots, hipStream_t st) {
    if (variant != QGEMV_VARIANT_MFMA && variant != QGEMV_VARIANT_MFMA_STAGED &&
        variant != QGEMV_VARIANT_MFMA_RESIDENT)
        return hipErrorNotSupported;
    // the kernel launch_small_m would run for this variant
    if ((variant == QGEMV_VARIANT_MFMA_RESIDENT && small_m3_supported(fmt, K, M)) ||
        (variant == QGEMV_VARIANT_MFMA && use_resident_kernel(fmt, N, K, M)))
        return launch_small_m3_dots(fmt, w, N, K, M, q, d, s, y, dots, st);
    if (variant != QGEMV_VARIANT_MFMA_STAGED && use_stream_kernel(fmt, N, M))
        return hipErrorNotSupported;   // the wave-stream kernel has no dots mode
    switch (fmt) {
    case QGEMV_FMT_Q4_K: return launch_mfma<QGEMV_FMT_Q4_K, true>(w, N, K, M, q, d, s, y, st, dots);
    case QGEMV_FMT_Q6_K: return launch_mfma<QGEMV_FMT_Q6_K, true>(w, N, K, M, q, d, s, y, st, dots);
    default: return launch_mfma<QGEMV_FMT_Q4_0, true>(w, N, K, M, q, d, s, y, st, dots);
    }
}

}  // namespace qgemv
