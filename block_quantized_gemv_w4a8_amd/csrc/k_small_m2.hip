// k_small_m2.hip -- the small-M product (a few activation rows, the prefill
// chunk) on the int8 matrix cores, with wave-private weight streams.
//
// Row m of y equals the batch-1 GEMV of activation row m (colibri GPU
// backends, eligibility gates: C = A x B is row-independent).  Where the work
// is a dense contraction the int8 matrix cores take it: each 32-wide K block
// gets its own exact int32 dot (Q6_K: each 16-group), because both the weights
// and the activation carry a scale per block, and the fp32 epilogue applies
// the scales ("Backends and hardware", section "CUDA": the prefill kernel's
// gap is staging the next weight tile behind the current multiply).
//
// Work split.  A workgroup of NW waves owns NTW tiles of 16 weight rows.  The
// waves of a tile split its 256-weight units (KSB ways, interleaved) and the
// four pairs of 32-blocks of every unit (KS ways).  Each wave streams its own
// weight bytes straight from HBM into registers, in the operand layout of
// v_mfma_i32_16x16x64_i8 (lane l: weight row l % 16, 16 K values of quarter
// l / 16 of a block pair), D units ahead of the one it multiplies; no other
// wave waits for them.  The activation (codes, and the fp16 scales and int32
// sums as they are stored) is shared: it moves through LDS in chunks of KC
// units, double-buffered, with one workgroup barrier per chunk.  Every thread
// loads its share of the next chunk into registers while the current one is
// computed and writes it to the other buffer before the barrier; the thread
// that brought a row's scales in writes them as fp32 (dx, and dx * s where
// the format has a min or offset term) in a [block][row] layout.
//
// Per 64-wide block pair a lane holds 16 weight codes; per activation tile of
// 16 rows, one 16-byte LDS read gives the A operand:
//   * M >= 9: one MFMA per block, the B operand masked to that block's K
//     lanes (quarters 0-1 are block 2p, 2-3 are block 2p+1);
//   * M <= 8 ("two-block" tiles): rows 0-7 of the A operand carry block 2p of
//     activation rows 0-7 (zeros in quarters 2-3) and rows 8-15 carry block
//     2p+1 (zeros in quarters 0-1), so one MFMA gives both blocks' dots for
//     eight rows and no tile row is wasted; rows m and m + 8 are added at the
//     end.
// Formats (per output element and block, fp32):
//   Q4_K  y += d*sc_j*dx*D  - (dmin*m_j)(dx*s)      codes 0..15
//   Q4_0  y += dw*dx*D      - (8*dw)(dx*s)          codes 0..15
//   Q6_K  y += d*(sc_g*D_g + sc_g'*D_g')*dx         codes - 32 as int8
// The second product of the first two lines is a small dense product over
// the blocks and goes to the fp32 MFMA.  For Q6_K the codes enter signed, so
// there is no offset term; the two 16-groups of a block are separate MFMAs
// (the other groups' K lanes zeroed), their int32 dots are scaled and added
// exactly in integers (|sc*D| < 2^23), and the unit's fp32 sum is scaled by d
// once.
#include <type_traits>

#include "qgemv_device.h"
#include "qgemv_launch.h"

namespace qgemv {
namespace sm2 {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Keeps the compiler from moving code, memory accesses included, across this
// point: the issue order of the loads is what the s_waitcnt counts assume,
// and hoisting a later unit's LDS reads above it only lengthens live ranges.
__device__ __forceinline__ void fence_code() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// The same for loads through the given restrict-qualified pointers, which a
// plain memory clobber does not hold: the compiler sank the activation-scale
// load, used only by the threads that write the scales, past it into that
// store at the end of the chunk, where its whole latency was then waited
// out.  Naming the pointers in the asm keeps every load of the chunk at its
// start (4096 x 14336, same process: 40.8 against 44.7 us at M = 64, 34.0
// against 40.2 us at M = 48, 29.9 against 35.8 us at M = 32; 12288 x 4096 at
// M = 64 37.5 against 41.7 us).
__device__ __forceinline__ void fence_loads(const void* a, const void* b, const void* c) {
    asm volatile("" ::"s"(a), "s"(b), "s"(c) : "memory");
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ i32x4 mfma64(const i32x4& a, const i32x4& b) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, i32x4{0, 0, 0, 0}, 0, 0, 0);
}

__device__ __forceinline__ i32x4 and4(const u32x4& v, uint32_t m) {
    return i32x4{(int)(v.x & m), (int)(v.y & m), (int)(v.z & m), (int)(v.w & m)};
}

// ------------------------------------------------------------ formats ----
// A unit is 256 consecutive weights of a row: a Q4_K super-block (144 B), a
// Q6_K super-block (210 B) or eight Q4_0 blocks (144 B).
template <int FMT>
struct Fmt;

// pw: the wave's first block pair (wave-uniform); BPW pairs from there.
template <>
struct Fmt<QGEMV_FMT_Q4_K> {
    static constexpr int UB = 144;
    static constexpr bool MIN = true;    // fp32 MFMA term with dx*s
    // vector-memory instructions of one unit's load (for s_waitcnt counts)
    template <int BPW> static constexpr int NLOAD = 1 + BPW;
    template <int BPW>
    struct W {
        u32x4 hdr;
        u32x4 qs[BPW];
    };
    template <int BPW>
    __device__ static __forceinline__ void load(const uint8_t* unit, int pw, int kq, W<BPW>& w) {
        w.hdr = *reinterpret_cast<const u32x4*>(unit);
#pragma unroll
        for (int i = 0; i < BPW; i++)
            w.qs[i] = *reinterpret_cast<const u32x4*>(unit + 16 + 32 * (pw + i) + 16 * (kq & 1));
    }
};

template <>
struct Fmt<QGEMV_FMT_Q6_K> {
    static constexpr int UB = 210;
    static constexpr bool MIN = false;
    // block pair p lies in half p / 2 of the super-block; the low nibbles of
    // its two blocks come from the same ql bytes (nibble p % 2) and the high
    // bit pairs from the same qh bytes: one ql and one qh load per half
    template <int BPW> static constexpr int NLOAD = 2 * ((BPW + 1) / 2) + BPW + 1;
    template <int BPW>
    struct W {
        u32x4 ql[(BPW + 1) / 2], qh[(BPW + 1) / 2];
        uint32_t sc[BPW];   // int8 scales of groups 4p .. 4p+3
        uint32_t d;
    };
    template <int BPW>
    __device__ static __forceinline__ void load(const uint8_t* unit, int pw, int kq, W<BPW>& w) {
#pragma unroll
        for (int i = 0; i < (BPW + 1) / 2; i++) {
            const int h = (pw + 2 * i) >> 1;
            w.ql[i] = ld16(unit + 64 * h + 32 * (kq >> 1) + 16 * (kq & 1));
            w.qh[i] = ld16(unit + 128 + 32 * h + 16 * (kq & 1));
        }
#pragma unroll
        for (int i = 0; i < BPW; i++)
            w.sc[i] = *reinterpret_cast<const uint32_t __attribute__((aligned(2)))*>(
                unit + 192 + 4 * (pw + i));
        w.d = ld2(unit + 208);
    }
};

template <>
struct Fmt<QGEMV_FMT_Q4_0> {
    static constexpr int UB = 144;
    static constexpr bool MIN = true;
    template <int BPW> static constexpr int NLOAD = 3 * BPW;
    template <int BPW>
    struct W {
        u32x4 qs[BPW];
        uint32_t d[BPW][2];
    };
    // nbl: blocks of the row from this unit on; a block past the row re-reads
    // the unit's first block (its scale is zeroed where it is used)
    template <int BPW>
    __device__ static __forceinline__ void load(const uint8_t* unit, int pw, int kq, int nbl,
                                                W<BPW>& w) {
#pragma unroll
        for (int i = 0; i < BPW; i++) {
            const int b = 2 * (pw + i) + (kq >> 1);
            w.qs[i] = ld16(unit + 18 * (b < nbl ? b : 0) + 2);
#pragma unroll
            for (int e = 0; e < 2; e++) {
                const int be = 2 * (pw + i) + e;
                w.d[i][e] = ld2(unit + 18 * (be < nbl ? be : 0));
            }
        }
    }
};

// Q6_K codes of one block pair for this lane, as signed bytes (code - 32):
// quarter kq of the pair is block 2p + kq/2, positions 16*(kq&1) .. +15; low
// nibble (p % 2) of ql, high bits at 4*(p % 2) + 2*(kq/2) of qh.
__device__ __forceinline__ u32x4 q6_codes(const u32x4& ql, const u32x4& qh, int par, int hsh) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t lo = (ql[i] >> (4 * par)) & LO4;
        const uint32_t hi = (qh[i] >> hsh) & 0x03030303u;
        const uint32_t x = (lo | (hi << 4)) ^ 0x20202020u;        // code - 32 mod 64
        const uint32_t s = x & 0x20202020u;                       // its sign bit
        r[i] = x | (s << 1) | (s << 2);                           // sign-extend to 8 bits
    }
    return r;
}

// ---------------------------------------------------------- the kernel ---

// LDS of one activation chunk (MP rows x KC units).  MPC code rows: MP, or
// 16 for the two-block tiles, whose rows MP .. 15 stay zero (the A-operand
// quarters of the other block read them).
template <int FMT, int MP, int MPC, int KC>
struct Chunk {
    static constexpr bool MIN = Fmt<FMT>::MIN;
    static constexpr int CSLOT = KC * 16 + 1;                 // 16-byte slots per code row (+1 pad)
    static constexpr int CSTR = 16 * CSLOT;                   // bytes per code row
    static constexpr int NCODE = MP * CSLOT;                  // code slots written per chunk
    static constexpr int NSC = MP * KC;                       // scale groups (row, 8 blocks)
    static constexpr int O_CODE = 0;
    static constexpr int O_DX = 16 * MPC * CSLOT;             // fp32 dx [KC*8][MP]
    static constexpr int O_DXS = O_DX + 4 * KC * 8 * MP;      // fp32 dx*s [KC*8][MP]
    static constexpr int BYTES = O_DXS + (MIN ? 4 * KC * 8 * MP : 0);
};

// FMT: weight format; MT: activation tiles of 16 rows; TWO: the two-block
// tiles (MT = 1, M <= 8); NTW: weight tiles per workgroup; KSB, KS: waves per
// tile over units and over block pairs; KC: units per activation chunk; D:
// units of weights in flight per wave; NW: waves per workgroup.
template <int FMT, int MT, bool TWO, int NTW, int KSB, int KS, int KC, int D, int NW>
__global__ __launch_bounds__(64 * NW) void k_small_m2(const uint8_t* __restrict__ w, int N, int K,
                                                  int M, const int8_t* __restrict__ q,
                                                  const uint16_t* __restrict__ dact,
                                                  const int32_t* __restrict__ sact,
                                                  float* __restrict__ y) {
    constexpr int NTH = 64 * NW;
    static_assert(NTW * KSB * KS == NW, "every wave has a tile, units and block pairs");
    static_assert(!TWO || MT == 1, "two-block tiles have one activation tile");
    static_assert(KC % KSB == 0, "every wave has units in every chunk");
    static_assert(KS == 1 || KS == 2 || KS == 4, "block pairs split evenly");
    using F = Fmt<FMT>;
    constexpr bool MIN = F::MIN;
    constexpr int MP = TWO ? 8 : 16 * MT;     // activation rows staged
    using C = Chunk<FMT, MP, TWO ? 16 : MP, KC>;
    static_assert(C::NSC <= NTH, "one scale group per thread");
    constexpr int BPW = 4 / KS;               // block pairs per wave and unit
    constexpr int SPC = KC / KSB;             // units per wave and chunk
    constexpr int NPART = KSB * KS;
    constexpr int NKK = BPW >= 2 ? BPW / 2 : 1;   // fp32-MFMA groups of 4 blocks per wave
    // Q6_K steps software-pipelined (below) where the registers allow: the
    // second set of MFMA results and both pairs' B operands spill at 16
    // waves (128 VGPRs)
    constexpr bool PIPE = FMT == QGEMV_FMT_Q6_K && !TWO && NW <= 8;
    // chunks per unrolled step: even (buffer parity) and a multiple of the
    // ring period
    constexpr int CU = (SPC % D == 0) ? 2 : ((2 * SPC) % D == 0 ? 2 : 2 * D);
    using W = typename F::template W<BPW>;

    __shared__ __align__(16) uint8_t buf0[C::BYTES];
    __shared__ __align__(16) uint8_t buf1[C::BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = wv / (KSB * KS), ksb = (wv / KS) % KSB, ks = wv % KS;
    const int part = ksb * KS + ks;
    const int pw = ks * BPW;                  // the wave's first block pair
    const int nl = lane & 15, kq = lane >> 4;
    const int Kp = (K + 255) / 256 * 256;
    const int nunits = Kp / 256, nb = Kp / 32;
    const int nbw = K / 32;
    const int nchunks = (nunits + KC - 1) / KC;
    const int64_t row_bytes = FMT == QGEMV_FMT_Q4_0 ? (int64_t)nbw * 18 : (int64_t)nunits * F::UB;
    const int n0 = blockIdx.x * (16 * NTW) + 16 * tile;
    const uint8_t* rowp = w + (int64_t)min(n0 + nl, N - 1) * row_bytes;

    if constexpr (TWO) {
        // code rows 8 .. 15 of both buffers: zeros
        for (int o = tid; o < 8 * C::CSTR / 16; o += NTH) {
            *reinterpret_cast<u32x4*>(buf0 + C::O_CODE + 8 * C::CSTR + 16 * o) = u32x4{0, 0, 0, 0};
            *reinterpret_cast<u32x4*>(buf1 + C::O_CODE + 8 * C::CSTR + 16 * o) = u32x4{0, 0, 0, 0};
        }
    }

    // ---- activation chunks, staged through registers: every thread loads
    // its 16-byte code slots and (one thread per scale group) 8 fp16 scales
    // and 8 sums of the next chunk while the current one is computed, and
    // writes them (the scales as fp32 dx and dx * s, [block][row]) before
    // the chunk barrier.  Loads are unconditional, with clamped addresses.
    constexpr int RC = (C::NCODE + NTH - 1) / NTH;         // code slots per thread
    int code_src[RC];                                      // row offset within q
    int code_piece[RC];                                    // byte offset within a chunk
#pragma unroll
    for (int r = 0; r < RC; r++) {
        const int s = min(r * NTH + tid, C::NCODE - 1);
        const int m = s / C::CSLOT;
        int pc = s - m * C::CSLOT;
        if (pc == KC * 16) pc = KC * 16 - 1;               // the pad slot re-reads its neighbour
        code_src[r] = min(m, M - 1) * Kp;
        code_piece[r] = 16 * pc;
    }
    const int sg = min(tid, C::NSC - 1);                    // this thread's scale group
    const int sg_m = sg / KC, sg_k = sg - (sg / KC) * KC;
    const int sg_row = min(sg_m, M - 1);
    struct ActRegs {
        u32x4 code[RC];
        u32x4 d;
        i32x4 sa, sb;
    };
    auto load_act = [&](int c, ActRegs& a) {
        const int kb = c * KC * 256;
#pragma unroll
        for (int r = 0; r < RC; r++) {
            const int off = min(kb + code_piece[r], Kp - 16);
            a.code[r] = *reinterpret_cast<const u32x4*>(q + code_src[r] + off);
        }
        const int blk = min((c * KC + sg_k) * 8, nb - 8);
        const int64_t g = (int64_t)sg_row * nb + blk;
        a.d = *reinterpret_cast<const u32x4*>(dact + g);
        if constexpr (MIN) {
            a.sa = *reinterpret_cast<const i32x4*>(sact + g);
            a.sb = *reinterpret_cast<const i32x4*>(sact + g + 4);
        }
    };
    auto store_act = [&](const ActRegs& a, uint8_t* b) {
#pragma unroll
        for (int r = 0; r < RC; r++) {
            const int s = r * NTH + tid;
            if (s < C::NCODE) *reinterpret_cast<u32x4*>(b + C::O_CODE + 16 * s) = a.code[r];
        }
        if (tid < C::NSC) {
            float* dx = reinterpret_cast<float*>(b + C::O_DX);
            float f[8];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                f[2 * j] = h2f(a.d[j] & 0xFFFFu);
                f[2 * j + 1] = h2f(a.d[j] >> 16);
            }
#pragma unroll
            for (int j = 0; j < 8; j++) dx[(8 * sg_k + j) * MP + sg_m] = f[j];
            if constexpr (MIN) {
                float* dxs = reinterpret_cast<float*>(b + C::O_DXS);
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    dxs[(8 * sg_k + j) * MP + sg_m] = f[j] * (float)a.sa[j];
                    dxs[(8 * sg_k + 4 + j) * MP + sg_m] = f[4 + j] * (float)a.sb[j];
                }
            }
        }
    };

    // ---- this wave's weight stream: its s-th unit
    auto unit_of = [&](int s) {
        const int c = s / SPC, i = s - (s / SPC) * SPC;
        return c * KC + ksb + KSB * i;
    };
    auto load_w = [&](int s, W& wr) {
        const int u = min(unit_of(s), nunits - 1);
        const uint8_t* up = rowp + (int64_t)F::UB * u;
        if constexpr (FMT == QGEMV_FMT_Q4_0) F::template load<BPW>(up, pw, kq, nbw - 8 * u, wr);
        else F::template load<BPW>(up, pw, kq, wr);
    };

    // accumulators: acc (block terms), acc2 (fp32-MFMA terms)
    f32x4 acc[MT], acc2[MT];
#pragma unroll
    for (int t = 0; t < MT; t++) {
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc2[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // lane constants
    const int hsh6 = 2 * (kq >> 1);                    // Q6_K: qh bit offset of this quarter
    const uint32_t m_lo = kq < 2 ? 0xFFFFFFFFu : 0u;   // quarters of block 2p
    const uint32_t m_hi = ~m_lo;
    // TWO: A rows 0-7 read block 2p (quarters 0-1), rows 8-15 block 2p+1
    // (quarters 2-3); the other quarters read the zero rows 8 .. 15
    const bool a_zero = TWO && ((nl < 8) != (kq < 2));
    const int a_row = TWO ? (nl & 7) + (a_zero ? 8 : 0) : nl;
    // fp32-MFMA term: K lane kq carries block 4kk + kq; with one block pair
    // per wave only the lanes of the wave's two blocks take part
    const bool mine = BPW >= 2 || (kq >> 1) == (pw & 1);
    // Per-lane byte offsets into a chunk buffer; the wave's units (ksb) and
    // block pairs (pw) are folded in here, so every LDS read of a unit is one
    // of these plus a constant (the unit's index i, the pair, the tile), which
    // the reads take as an immediate offset.
    const int a_off = C::O_CODE + a_row * C::CSTR + 16 * kq + 256 * ksb + 64 * pw;
    const int x_off = C::O_DX + 4 * ((8 * ksb + 2 * pw) * MP +
                                     (TWO ? (kq >> 1) * MP + 4 * (kq & 1) : 4 * kq));
    const int xs_off = C::O_DXS + 4 * ((8 * ksb + 4 * (pw / 2) + kq) * MP + (TWO ? (nl & 7) : nl));

    // the i-th unit of this wave in the chunk (unit ksb + KSB * i of it), from
    // registers wr and the chunk in LDS b; nbl: blocks of the row from this
    // unit on (<= 0: the unit is past the row and adds zeros)
    auto compute = [&](const W& wr, int i, const uint8_t* b, int nbl) {
        const bool valid = nbl > 0;
        const uint8_t* codes = b + a_off + 256 * KSB * i;
        const uint8_t* dxT = b + x_off + 4 * 8 * KSB * i * MP;
        const uint8_t* dxsT = b + xs_off + 4 * 8 * KSB * i * MP;
        float fd = 0.f, fdm = 0.f;
        uint32_t slo = 0, shi = 0, mlo = 0, mhi = 0;
        if constexpr (FMT == QGEMV_FMT_Q4_K) {
            fd = valid ? h2f(wr.hdr.x & 0xFFFFu) : 0.0f;
            fdm = valid ? h2f(wr.hdr.x >> 16) : 0.0f;
            slo = wr.hdr.y & 0x3F3F3F3Fu;
            shi = (wr.hdr.w & LO4) | ((wr.hdr.y >> 2) & 0x30303030u);
            mlo = wr.hdr.z & 0x3F3F3F3Fu;
            mhi = ((wr.hdr.w >> 4) & LO4) | ((wr.hdr.z >> 2) & 0x30303030u);
        } else if constexpr (FMT == QGEMV_FMT_Q6_K) {
            fd = valid ? h2f(wr.d) : 0.0f;
        }
        f32x4 accs[MT];   // Q6_K: the unit's sum before the d scale
        if constexpr (FMT == QGEMV_FMT_Q6_K) {
#pragma unroll
            for (int t = 0; t < MT; t++) accs[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if constexpr (PIPE) {
            // The (block pair, activation tile) steps of the unit run as one
            // software pipeline: step k's MFMAs and the LDS reads of its
            // scales and of step k+1's codes issue before step k-1's
            // epilogue, one MFMA between every few of its VALU instructions,
            // so neither the LDS nor the MFMA latency is waited out (the
            // register fence closing each epilogue would otherwise hold every
            // later LDS read behind it).  Both pairs' B operands are unpacked
            // first, so the pipeline runs through the pair boundary.  On 4096
            // x 14336: 45.7 against 48.3 us at M = 64, 40.6 against 42.7 us
            // at M = 48, 36.0 against 37.5 us at M = 32 for a pipeline within
            // each pair (same process), and 44.6, 40.0 and 35.6 us through
            // the pair boundary; 12288 x 4096 at M = 64 41.5 against 46.1
            // us, 128256 x 4096 at M = 64 324 against 355 us.
            i32x4 Bq[BPW][4];
            int scq[BPW][4];
#pragma unroll
            for (int pi = 0; pi < BPW; pi++) {
                const int p = pw + pi;
                const u32x4 c = q6_codes(wr.ql[pi / 2], wr.qh[pi / 2], p & 1, 4 * (p & 1) + hsh6);
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    Bq[pi][g] = and4(c, kq == g ? 0xFFFFFFFFu : 0u);
                    scq[pi][g] = sbyte(wr.sc[pi], g);
                }
            }
            constexpr int NK = BPW * MT;
            auto ld_a = [&](int k) {
                const int pi = k / MT, t = k % MT;
                const u32x4 av = *reinterpret_cast<const u32x4*>(codes + 16 * t * C::CSTR + 64 * pi);
                return i32x4{(int)av.x, (int)av.y, (int)av.z, (int)av.w};
            };
            auto ld_x = [&](int k, int h) {
                const int pi = k / MT, t = k % MT;
                return *reinterpret_cast<const f32x4*>(dxT + 4 * ((2 * pi + h) * MP + 16 * t));
            };
            auto epi = [&](int k, const i32x4 (&Dv)[4], const f32x4& x0, const f32x4& x1) {
                const int pi = k / MT, t = k % MT;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int v0 = __mul24(Dv[0][e], scq[pi][0]) + __mul24(Dv[1][e], scq[pi][1]);
                    const int v1 = __mul24(Dv[2][e], scq[pi][2]) + __mul24(Dv[3][e], scq[pi][3]);
                    const float a = fmaf((float)v0, x0[e], accs[t][e]);
                    accs[t][e] = fmaf((float)v1, x1[e], a);
                }
                asm volatile("" : "+v"(accs[t]));
            };
            i32x4 A = ld_a(0);
            i32x4 Dp[4];
            f32x4 xp0, xp1;
#pragma unroll
            for (int k = 0; k < NK; k++) {
                i32x4 Dc[4];
#pragma unroll
                for (int g = 0; g < 4; g++) Dc[g] = mfma64(A, Bq[k / MT][g]);
                const f32x4 xc0 = ld_x(k, 0), xc1 = ld_x(k, 1);
                if (k + 1 < NK) A = ld_a(k + 1);
                if (k > 0) epi(k - 1, Dp, xp0, xp1);
                // issue order (scheduler group masks: 0x008 MFMA, 0x100 LDS
                // read, 0x002 VALU): MFMA, the three LDS reads, six VALU,
                // then each further MFMA followed by six VALU
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
#pragma unroll
                for (int g = 1; g < 4; g++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int g = 0; g < 4; g++) Dp[g] = Dc[g];
                xp0 = xc0;
                xp1 = xc1;
            }
            epi(NK - 1, Dp, xp0, xp1);
        }
#pragma unroll
        for (int pi = 0; pi < (PIPE ? 0 : BPW); pi++) {
            // block pairs one after another: interleaving them only raises
            // the register count (the waves of a SIMD hide the latencies)
            if (pi > 0) __builtin_amdgcn_sched_barrier(0);
            const int p = pw + pi;                     // block pair (wave-uniform)
            const int j0 = 2 * p;                      // its first block
            // B operands
            i32x4 Bop[4];
            if constexpr (FMT == QGEMV_FMT_Q6_K) {
                const u32x4 c = q6_codes(wr.ql[pi / 2], wr.qh[pi / 2], p & 1, 4 * (p & 1) + hsh6);
                if constexpr (TWO) {
                    // groups: even quarters (0, 2), then odd quarters (1, 3)
                    const uint32_t me = (kq & 1) ? 0u : 0xFFFFFFFFu;
                    Bop[0] = and4(c, me);
                    Bop[1] = and4(c, ~me);
                } else {
#pragma unroll
                    for (int g = 0; g < 4; g++) Bop[g] = and4(c, kq == g ? 0xFFFFFFFFu : 0u);
                }
            } else {
                // Q4_K: quarters 0-1 low nibbles (block 2p), 2-3 high (block
                // 2p+1); Q4_0: quarter kq is nibble kq&1 of block 2p + kq/2
                const int sh = FMT == QGEMV_FMT_Q4_K ? 4 * (kq >> 1) : 4 * (kq & 1);
                u32x4 c;
#pragma unroll
                for (int e = 0; e < 4; e++) c[e] = (wr.qs[pi][e] >> sh) & LO4;
                if constexpr (TWO) {
                    Bop[0] = and4(c, 0xFFFFFFFFu);
                } else {
                    Bop[0] = and4(c, m_lo);
                    Bop[1] = and4(c, m_hi);
                }
            }
            // weight scales of the pair's blocks (per lane: its row; TWO:
            // the block of the lane's output rows)
            float ws[2];
            int sc6[4];
            if constexpr (FMT == QGEMV_FMT_Q4_K) {
                const uint32_t sb = j0 >= 4 ? shi : slo;
                if constexpr (TWO) {
                    ws[0] = fd * (float)bfe(sb, 8 * ((j0 & 3) + (kq >> 1)), 8);
                } else {
                    ws[0] = fd * (float)bfe(sb, 8 * (j0 & 3), 8);
                    ws[1] = fd * (float)bfe(sb, 8 * (j0 & 3) + 8, 8);
                }
            } else if constexpr (FMT == QGEMV_FMT_Q4_0) {
                const bool v0 = j0 < nbl, v1 = j0 + 1 < nbl;
                if constexpr (TWO) {
                    const bool vv = (kq < 2) ? v0 : v1;
                    ws[0] = vv ? h2f(kq < 2 ? wr.d[pi][0] : wr.d[pi][1]) : 0.0f;
                } else {
                    ws[0] = v0 ? h2f(wr.d[pi][0]) : 0.0f;
                    ws[1] = v1 ? h2f(wr.d[pi][1]) : 0.0f;
                }
            } else {
                const uint32_t sw = wr.sc[pi];   // int8 scales of groups 4p .. 4p+3
                if constexpr (TWO) {
                    const int e = kq >> 1;   // block of this lane's rows
                    sc6[0] = sbyte(sw, 2 * e);
                    sc6[1] = sbyte(sw, 2 * e + 1);
                } else {
#pragma unroll
                    for (int g = 0; g < 4; g++) sc6[g] = sbyte(sw, g);
                }
            }
#pragma unroll
            for (int t = 0; t < MT; t++) {
                // A operand: 16 codes of rows 16t + l%16 (TWO: see a_row)
                const u32x4 av =
                    *reinterpret_cast<const u32x4*>(codes + 16 * t * C::CSTR + 64 * pi);
                const i32x4 A = {(int)av.x, (int)av.y, (int)av.z, (int)av.w};
                if constexpr (TWO) {
                    // output rows 4kq+i: kq < 2 -> block j0 (rows 4kq+i), kq >= 2
                    // -> block j0+1 (rows 4kq-8+i)
                    const f32x4 x4 = *reinterpret_cast<const f32x4*>(dxT + 4 * 2 * pi * MP);
                    if constexpr (FMT == QGEMV_FMT_Q6_K) {
                        const i32x4 De = mfma64(A, Bop[0]);
                        const i32x4 Do = mfma64(A, Bop[1]);
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            const int v = __mul24(De[e], sc6[0]) + __mul24(Do[e], sc6[1]);
                            accs[t][e] = fmaf((float)v, x4[e], accs[t][e]);
                        }
                    } else {
                        const i32x4 Dd = mfma64(A, Bop[0]);
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            acc[t][e] = fmaf((float)Dd[e], ws[0] * x4[e], acc[t][e]);
                    }
                } else {
                    const f32x4 x0 =
                        *reinterpret_cast<const f32x4*>(dxT + 4 * (2 * pi * MP + 16 * t));
                    const f32x4 x1 =
                        *reinterpret_cast<const f32x4*>(dxT + 4 * ((2 * pi + 1) * MP + 16 * t));
                    if constexpr (FMT == QGEMV_FMT_Q6_K) {
                        const i32x4 D0 = mfma64(A, Bop[0]);
                        const i32x4 D1 = mfma64(A, Bop[1]);
                        const i32x4 D2 = mfma64(A, Bop[2]);
                        const i32x4 D3 = mfma64(A, Bop[3]);
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            const int v0 = __mul24(D0[e], sc6[0]) + __mul24(D1[e], sc6[1]);
                            const int v1 = __mul24(D2[e], sc6[2]) + __mul24(D3[e], sc6[3]);
                            const float a = fmaf((float)v0, x0[e], accs[t][e]);
                            accs[t][e] = fmaf((float)v1, x1[e], a);
                        }
                    } else {
                        const i32x4 D0 = mfma64(A, Bop[0]);
                        const i32x4 D1 = mfma64(A, Bop[1]);
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            const float a = fmaf((float)D0[e], ws[0] * x0[e], acc[t][e]);
                            acc[t][e] = fmaf((float)D1[e], ws[1] * x1[e], a);
                        }
                    }
                }
                // the pair's epilogue is done here: without this the compiler
                // computes every MFMA of a step first and holds the results
                if constexpr (FMT == QGEMV_FMT_Q6_K) asm volatile("" : "+v"(accs[t]));
                else asm volatile("" : "+v"(acc[t]));
            }
        }
        if constexpr (FMT == QGEMV_FMT_Q6_K) {
#pragma unroll
            for (int t = 0; t < MT; t++) {
#pragma unroll
                for (int e = 0; e < 4; e++) acc[t][e] = fmaf(fd, accs[t][e], acc[t][e]);
                asm volatile("" : "+v"(acc[t]));
            }
        }
        if constexpr (MIN) {
            // the fp32-MFMA terms: K lane kq of the MFMA carries block
            // 4kk + kq of the wave's blocks
#pragma unroll
            for (int g = 0; g < NKK; g++) {
                float bm;
                if constexpr (FMT == QGEMV_FMT_Q4_K) {
                    const int kk = pw / 2 + g;       // wave-uniform
                    const uint32_t mb = kk ? mhi : mlo;
                    bm = mine ? fdm * (float)bfe(mb, 8 * kq, 8) : 0.0f;
                } else {
                    // 8 * dw of block 4kk + kq: the wave's pair 2g + kq/2
                    // (one pair per wave: its pair), element kq & 1
                    const int lp = BPW >= 2 ? 2 * g + (kq >> 1) : 0;
                    uint32_t dv = wr.d[0][0];
#pragma unroll
                    for (int pi = 0; pi < BPW; pi++)
#pragma unroll
                        for (int e = 0; e < 2; e++)
                            if (pi == lp && e == (kq & 1)) dv = wr.d[pi][e];
                    const int blk = 2 * (pw + lp) + (kq & 1);
                    bm = (mine && blk < nbl) ? 8.0f * h2f(dv) : 0.0f;
                }
#pragma unroll
                for (int t = 0; t < MT; t++) {
                    float a = *reinterpret_cast<const float*>(dxsT + 4 * (4 * g * MP + 16 * t));
                    if (TWO && nl >= 8) a = 0.0f;
                    acc2[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bm, acc2[t], 0, 0, 0);
                    asm volatile("" : "+v"(acc2[t]));
                }
            }
        }
    };

    // ---- prologue: chunk 0 and the first D units of weights
    {
        ActRegs a0;
        load_act(0, a0);
        store_act(a0, buf0);
    }
    W ring[D];
#pragma unroll
    for (int r = 0; r < D; r++) load_w(r, ring[r]);
    __syncthreads();

    // ---- main loop: CU chunks per step, ring slot and buffer constant.
    // Nothing in it is conditional: a chunk past the last one (the step's
    // remainder) and units past the row are computed on re-read valid bytes
    // with their scales zeroed, and the chunk loads of the last chunk repeat
    // it; a branch around loads or their uses makes the compiler wait for
    // every load in flight.  The barrier orders LDS only, so the weights in
    // flight stay in flight across it (a __syncthreads() would wait for
    // them).
    const int nsteps = (nchunks + CU - 1) / CU;
    for (int st = 0; st < nsteps; st++) {
#pragma unroll
        for (int cc = 0; cc < CU; cc++) {
            const int c = st * CU + cc;
            uint8_t* cur = (cc & 1) ? buf1 : buf0;
            uint8_t* nxt = (cc & 1) ? buf0 : buf1;
            ActRegs an;
            load_act(min(c + 1, nchunks - 1), an);
            fence_loads(q, dact, sact);
#pragma unroll
            for (int i = 0; i < SPC; i++) {
                const int s = c * SPC + i;
                const int rs = (cc * SPC + i) % D;
                const int u = c * KC + ksb + KSB * i;
                compute(ring[rs], i, cur, nbw - 8 * u);
                fence_code();
                load_w(s + D, ring[rs]);
                fence_code();
            }
            store_act(an, nxt);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        }
    }

    // ---- partial sums of the waves of a tile meet in LDS (buf0 is free
    // after the last barrier), added in part order
    float* pbuf = reinterpret_cast<float*>(buf0);
    static_assert(NTW * NPART * MT * 4 * 64 * 4 <= C::BYTES, "partials fit");
#pragma unroll
    for (int t = 0; t < MT; t++)
#pragma unroll
        for (int e = 0; e < 4; e++)
            pbuf[(((tile * NPART + part) * MT + t) * 4 + e) * 64 + lane] = acc[t][e] - acc2[t][e];
    __syncthreads();
    const int nout = NTW * 16 * M;
    for (int o = tid; o < nout; o += NTH) {
        const int m = o / (NTW * 16), nloc = o - (o / (NTW * 16)) * (NTW * 16);
        const int tl = nloc >> 4, ln = nloc & 15;
        const int n = blockIdx.x * (16 * NTW) + nloc;
        if (n >= N) continue;
        float v = 0.0f;
        if constexpr (TWO) {
            // row m: lanes of quarter m/4 (block 2p) and m/4 + 2 (block 2p+1)
            const int e = m & 3, l0 = 16 * (m >> 2) + ln, l1 = l0 + 32;
            float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
            for (int pp = 0; pp < NPART; pp++) {
                v0 += pbuf[((tl * NPART + pp) * 4 + e) * 64 + l0];
                v1 += pbuf[((tl * NPART + pp) * 4 + e) * 64 + l1];
            }
            v = v0 + v1;
        } else {
            const int t = m >> 4, r = m & 15, e = r & 3, l = 16 * (r >> 2) + ln;
#pragma unroll
            for (int pp = 0; pp < NPART; pp++)
                v += pbuf[(((tl * NPART + pp) * MT + t) * 4 + e) * 64 + l];
        }
        y[(int64_t)m * N + n] = v;
    }
}

template <int FMT, int MT, bool TWO, int NTW, int KSB, int KS, int KC, int D, int NW = 8>
static hipError_t launch_cfg(const void* w, int64_t N, int64_t K, int64_t M, const int8_t* q,
                             const uint16_t* d, const int32_t* s, float* y, hipStream_t st) {
    const int64_t grid = (N + 16 * NTW - 1) / (16 * NTW);
    launch_kernel((k_small_m2<FMT, MT, TWO, NTW, KSB, KS, KC, D, NW>), dim3((unsigned)grid),
                  dim3(64 * NW), 0, st, (const uint8_t*)w, (int)N, (int)K, (int)M, q, d, s, y);
    return hipGetLastError();
}

// Matrices with fewer 16-row tiles than this split the units of a tile over
// more waves instead of giving a workgroup several tiles.
constexpr int64_t kWideTiles = 512;

template <int FMT>
static hipError_t launch_fmt(const void* w, int64_t N, int64_t K, int64_t M, const int8_t* q,
                             const uint16_t* d, const int32_t* s, float* y, hipStream_t st) {
    const bool wide = (N + 15) / 16 >= kWideTiles;
    const int mt = (int)((M + 15) / 16);
    // <FMT, MT, TWO, NTW, KSB, KS, KC, D>
    if (wide) {
        if (M <= 8) return launch_cfg<FMT, 1, true, 4, 2, 1, 8, 4>(w, N, K, M, q, d, s, y, st);
        // Q6_K at M = 17-64: four tiles per 8-wave workgroup, each tile's
        // units split 2 ways, whole units per wave, one unit in flight per
        // wave, 4 units per activation chunk up to M = 48 and 2 at M = 49-64
        // (4 spill there).  Against the earlier two tiles per 16-wave
        // workgroup with units split 4 ways and block pairs 2 ways (same
        // process): 12288 x 4096 at M = 24 27.1 against 32.9 us, at M = 32
        // 27.4 against 33.2 us, at M = 48 32.2 against 37.8 us; 128256 x 4096
        // at M = 32 206 against 255 us, at M = 48 238 against 289 us.  At M =
        // 49-64: 46.2 against 48.9 us for two units in flight on 12288 x
        // 4096, 355 against 375 us on 128256 x 4096 (before the pipelined
        // steps)
        if constexpr (FMT == QGEMV_FMT_Q6_K) {
            if (mt == 2) return launch_cfg<FMT, 2, false, 4, 2, 1, 4, 1>(w, N, K, M, q, d, s, y, st);
            if (mt == 3) return launch_cfg<FMT, 3, false, 4, 2, 1, 4, 1>(w, N, K, M, q, d, s, y, st);
            if (mt >= 4) return launch_cfg<FMT, 4, false, 4, 2, 1, 2, 1>(w, N, K, M, q, d, s, y, st);
        }
        switch (mt) {
        case 1: return launch_cfg<FMT, 1, false, 4, 2, 1, 8, 4>(w, N, K, M, q, d, s, y, st);
        case 2: return launch_cfg<FMT, 2, false, 4, 2, 1, 4, 4>(w, N, K, M, q, d, s, y, st);
        case 3: return launch_cfg<FMT, 3, false, 4, 2, 1, 2, 2>(w, N, K, M, q, d, s, y, st);
        default: return launch_cfg<FMT, 4, false, 4, 2, 1, 2, 2>(w, N, K, M, q, d, s, y, st);
        }
    }
    if (M <= 8) return launch_cfg<FMT, 1, true, 1, 2, 4, 8, 4>(w, N, K, M, q, d, s, y, st);
    // Q6_K at M = 17-64: a tile's units split 4 ways and its block pairs 2
    // ways, 4 units per activation chunk, one unit in flight per wave.  On
    // 4096 x 14336 (same process): M = 64 48.3 against 63.5 us (units 2
    // ways, block pairs 4 ways, two units in flight) and against 54.2 us
    // with 16 waves; M = 48 42.7 against 59.5 us; M = 24 37.3 against 38.3
    // us for the staged kernel
    if constexpr (FMT == QGEMV_FMT_Q6_K) {
        if (mt == 2) return launch_cfg<FMT, 2, false, 1, 4, 2, 4, 1>(w, N, K, M, q, d, s, y, st);
        if (mt == 3) return launch_cfg<FMT, 3, false, 1, 4, 2, 4, 1>(w, N, K, M, q, d, s, y, st);
        if (mt >= 4) return launch_cfg<FMT, 4, false, 1, 4, 2, 4, 1>(w, N, K, M, q, d, s, y, st);
    }
    switch (mt) {
    case 1: return launch_cfg<FMT, 1, false, 1, 2, 4, 8, 4>(w, N, K, M, q, d, s, y, st);
    case 2: return launch_cfg<FMT, 2, false, 1, 2, 4, 4, 4>(w, N, K, M, q, d, s, y, st);
    case 3: return launch_cfg<FMT, 3, false, 1, 2, 4, 2, 2>(w, N, K, M, q, d, s, y, st);
    default: return launch_cfg<FMT, 4, false, 1, 2, 4, 2, 2>(w, N, K, M, q, d, s, y, st);
    }
}

}  // namespace sm2

hipError_t launch_small_m2(int fmt, const void* w, int64_t N, int64_t K, int64_t M,
                           const int8_t* q, const uint16_t* d, const int32_t* s, float* y,
                           hipStream_t st) {
    switch (fmt) {
    case QGEMV_FMT_Q4_K: return sm2::launch_fmt<QGEMV_FMT_Q4_K>(w, N, K, M, q, d, s, y, st);
    case QGEMV_FMT_Q6_K: return sm2::launch_fmt<QGEMV_FMT_Q6_K>(w, N, K, M, q, d, s, y, st);
    default: return sm2::launch_fmt<QGEMV_FMT_Q4_0>(w, N, K, M, q, d, s, y, st);
    }
}

}  // namespace qgemv
