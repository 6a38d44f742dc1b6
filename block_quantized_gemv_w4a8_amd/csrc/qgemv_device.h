// qgemv_device.h -- device-side building blocks shared by every kernel of
// libqgemv: unaligned byte loads, the 4 x int8 dot, and per-format "units".
//
// A unit is 64 consecutive weights of one row (the same for every format), so
// that one lane always pairs with 64 activation codes = 16 dwords:
//   Q4_K : unit u = chunk c (0..3) of super-block S = u/4; its 32 packed bytes
//          hold sub-blocks 2c (low nibbles) and 2c+1 (high nibbles); the
//          super-block header (d, dmin, 12 scale bytes) is read alongside.
//   Q6_K : unit u = quarter (h, t) of super-block S = u/4 (h = half, t = which
//          16 of the 32 positions l): 16 B of low nibbles for positions l,
//          16 B for l+32, 16 B of high bit pairs; that is 4 complete groups of
//          16 weights (elements 128h + 16t + 32j + 0..15, j = 0..3).
//   Q4_0 / Q8_0 : unit u = blocks 2u and 2u+1 (the second may be absent when
//          the row has an odd number of blocks).
// The unit loaders read the packed bytes straight from global memory, and the
// unit dot functions turn them into exact int32 block dots; the GEMV, the
// small-M and the block-dots kernels all call these same functions.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace qgemv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Loads of packed weight bytes.  The vector types carry 2-byte alignment so
// that one dwordx4 / dwordx2 load is emitted even where the address is only
// 2-byte aligned (Q6_K super-blocks start at 210*S, Q4_0 blocks at 18*b); the
// HSA runtime runs the memory system in unaligned mode.  These are ordinary
// (temporal) loads on purpose: one wave instruction covers only part of each
// cache line and sibling instructions read the rest, so the line has to stay
// in cache until they do (a non-temporal hint made the lines re-fetch).
typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
typedef uint32_t u32x2_a2 __attribute__((ext_vector_type(2), aligned(2)));

__device__ __forceinline__ u32x4 ld16(const uint8_t* p) {
    const u32x4_a2 v = *reinterpret_cast<const u32x4_a2*>(p);
    return u32x4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ u32x2 ld8(const uint8_t* p) {
    const u32x2_a2 v = *reinterpret_cast<const u32x2_a2*>(p);
    return u32x2{v.x, v.y};
}
__device__ __forceinline__ uint32_t ld2(const uint8_t* p) {
    return *reinterpret_cast<const uint16_t*>(p);
}

// A 16-byte chunk of a weight row for the LDS-staged kernels: one wave
// instruction covers 1 KB of consecutive bytes, so whole cache lines are
// consumed by one instruction and the non-temporal hint is safe there.
template <bool NT>
__device__ __forceinline__ u32x4 ld16_stream(const uint8_t* p) {
    const u32x4_a2 v = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_a2*>(p))
                          : *reinterpret_cast<const u32x4_a2*>(p);
    return u32x4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ void st16(uint8_t* p, u32x4 v) {
    *reinterpret_cast<u32x4_a2*>(p) = u32x4_a2{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ float h2f(uint32_t bits) {
    return __half2float(__ushort_as_half((unsigned short)bits));
}

// Signed 4 x int8 dot with int32 accumulate (v_dot4_i32_i8).
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

__device__ __forceinline__ uint32_t bfe(uint32_t x, uint32_t off, uint32_t w) {
    return __builtin_amdgcn_ubfe(x, off, w);
}

__device__ __forceinline__ int sbyte(uint32_t x, uint32_t k) {
    return __builtin_amdgcn_sbfe((int)x, 8 * k, 8);
}

constexpr uint32_t LO4 = 0x0F0F0F0Fu;

// LDS field readers.  Fields that sit 2 bytes off a 4-byte boundary are read
// as aligned dwords and shifted into place with v_alignbyte: unaligned LDS
// accesses stall the LDS pipeline on this chip, aligned dword reads do not.
__device__ __forceinline__ u32x4 lds16(const uint8_t* base, int off) {
    return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ __forceinline__ uint32_t lds2(const uint8_t* base, int off) {
    return *reinterpret_cast<const uint16_t*>(base + off);
}
__device__ __forceinline__ uint32_t abyte(uint32_t hi, uint32_t lo, uint32_t sh) {
    return __builtin_amdgcn_alignbyte(hi, lo, sh);
}
// 16 bytes at any even LDS offset (reads up to 4 bytes past the field).
__device__ __forceinline__ u32x4 lds16_a2(const uint8_t* base, int off) {
    const uint32_t* d = reinterpret_cast<const uint32_t*>(base + (off & ~3));
    const uint32_t sh = off & 3;
    const uint32_t w0 = d[0], w1 = d[1], w2 = d[2], w3 = d[3], w4 = d[4];
    return u32x4{abyte(w1, w0, sh), abyte(w2, w1, sh), abyte(w3, w2, sh), abyte(w4, w3, sh)};
}
// 8 bytes at any even LDS offset.
__device__ __forceinline__ u32x2 lds8_a2(const uint8_t* base, int off) {
    const uint32_t* d = reinterpret_cast<const uint32_t*>(base + (off & ~3));
    const uint32_t sh = off & 3;
    const uint32_t w0 = d[0], w1 = d[1], w2 = d[2];
    return u32x2{abyte(w1, w0, sh), abyte(w2, w1, sh)};
}

// Activation view of one unit: 16 dwords of codes (elements 64u .. 64u+63 of
// the activation row, as laid out for the weights of the format).
struct Act16 {
    uint32_t a[16];
};

// ------------------------------------------------------------------ Q4_K --
struct Q4K {
    static constexpr int SB_BYTES = 144;
    static constexpr int NDOT = 2;  // int32 dots per unit (sub-blocks 2c, 2c+1)
    struct W {
        u32x4 hdr, qa, qb;
    };
    __device__ static __forceinline__ void load(const uint8_t* row, int u, W& w) {
        const uint8_t* p = row + SB_BYTES * (u >> 2);
        const int c = u & 3;
        w.hdr = ld16(p);
        w.qa = ld16(p + 16 + 32 * c);
        w.qb = ld16(p + 32 + 32 * c);
    }
    // Unpacked codes of a unit: lo = sub-block 2c (elements 64u + 0..31),
    // hi = sub-block 2c+1 (elements 64u + 32..63), 4 codes per dword.
    struct C {
        uint32_t lo[8], hi[8];
    };
    __device__ static __forceinline__ void unpack(const W& w, C& c) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            c.lo[i] = w.qa[i] & LO4;
            c.lo[4 + i] = w.qb[i] & LO4;
            c.hi[i] = (w.qa[i] >> 4) & LO4;
            c.hi[4 + i] = (w.qb[i] >> 4) & LO4;
        }
    }
    // Activation elements of unit u start at 64u: sub-block 2c is a[0..7],
    // sub-block 2c+1 is a[8..15].
    __device__ static __forceinline__ void dots_c(const C& c, const Act16& x, int D[2]) {
        int d0 = 0, d1 = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            d0 = dot4(c.lo[i], x.a[i], d0);
            d1 = dot4(c.hi[i], x.a[8 + i], d1);
        }
        D[0] = d0;
        D[1] = d1;
    }
    __device__ static __forceinline__ void dots(const W& w, const Act16& x, int D[2]) {
        C c;
        unpack(w, c);
        dots_c(c, x, D);
    }
    // 6-bit scale and min of sub-block j (0..7) from the 12 header bytes
    // b[0..11] = hdr.y, hdr.z, hdr.w:
    //   j < 4 : scale = b[j] & 63, min = b[j+4] & 63
    //   j >= 4: scale = (b[j+4] & 15) | (b[j-4] >> 6) << 4,
    //           min   = (b[j+4] >> 4) | (b[j]   >> 6) << 4
    __device__ static __forceinline__ void scale_min(const W& w, int j, int& sc, int& mn) {
        if (j < 4) {
            sc = (int)bfe(w.hdr.y, 8 * j, 6);
            mn = (int)bfe(w.hdr.z, 8 * j, 6);
        } else {
            const uint32_t k = j - 4;
            sc = (int)(bfe(w.hdr.w, 8 * k, 4) | (bfe(w.hdr.y, 8 * k + 6, 2) << 4));
            mn = (int)(bfe(w.hdr.w, 8 * k + 4, 4) | (bfe(w.hdr.z, 8 * k + 6, 2) << 4));
        }
    }
};

// ------------------------------------------------------------------ Q6_K --
struct Q6K {
    static constexpr int SB_BYTES = 210;
    static constexpr int NDOT = 4;  // int32 dots per unit (4 groups of 16)
    struct W {
        u32x4 qa, qb, qh;
        u32x2 sc;
        uint32_t d;
    };
    __device__ static __forceinline__ void load(const uint8_t* row, int u, W& w) {
        const uint8_t* p = row + SB_BYTES * (u >> 2);
        const int h = (u >> 1) & 1, t = u & 1;
        w.qa = ld16(p + 64 * h + 16 * t);        // ql[64h + 16t ..]: positions l
        w.qb = ld16(p + 64 * h + 32 + 16 * t);   // ql[64h + 32 + 16t ..]: l + 32
        w.qh = ld16(p + 128 + 32 * h + 16 * t);  // qh[32h + 16t ..]
        w.sc = ld8(p + 192 + 8 * h);             // scales of groups 8h .. 8h+7
        w.d = ld2(p + 208);
    }
    // The repacked layout (QGEMV_FMT_Q6_K_R8): a row is tiles of 8
    // super-blocks, each tile 1680 bytes = ql[8][128] | qh[8][64] | sc[8][16]
    // | d[8] (fp16); super-block i of a tile keeps its bytes, only moved, so
    // every field of a unit starts on a 16-byte (sc: 8-byte) boundary.
    static constexpr int TILE_SB = 8, TILE_BYTES = 1680;
    static constexpr int T_QH = 1024, T_SC = 1536, T_D = 1664;
    __device__ static __forceinline__ void load_r8(const uint8_t* row, int u, W& w) {
        const int S = u >> 2, i = S & 7;
        const uint8_t* p = row + TILE_BYTES * (S >> 3);
        const int h = (u >> 1) & 1, t = u & 1;
        w.qa = ld16(p + 128 * i + 64 * h + 16 * t);
        w.qb = ld16(p + 128 * i + 64 * h + 32 + 16 * t);
        w.qh = ld16(p + T_QH + 64 * i + 32 * h + 16 * t);
        w.sc = ld8(p + T_SC + 16 * i + 8 * h);
        w.d = ld2(p + T_D + 2 * i);
    }
    // Activation of unit u = quarter (h, t): group j (elements
    // 128h + 16t + 32j + 0..15 of the super-block) is a[4j .. 4j+3].
    // init[j] = -32 * (sum of those 16 activation codes) folds the code offset
    // into the dot's accumulator, so D16_j = sum (code - 32) * q exactly.
    __device__ static __forceinline__ void dots(const W& w, const Act16& x, const int init[4],
                                                int D[4]) {
        int d0 = init[0], d1 = init[1], d2 = init[2], d3 = init[3];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t qa = w.qa[i], qb = w.qb[i], qh = w.qh[i];
            const uint32_t c0 = (qa & LO4) | ((qh << 4) & 0x30303030u);
            const uint32_t c1 = (qb & LO4) | ((qh << 2) & 0x30303030u);
            const uint32_t c2 = ((qa >> 4) & LO4) | (qh & 0x30303030u);
            const uint32_t c3 = ((qb >> 4) & LO4) | ((qh >> 2) & 0x30303030u);
            d0 = dot4(c0, x.a[i], d0);
            d1 = dot4(c1, x.a[4 + i], d1);
            d2 = dot4(c2, x.a[8 + i], d2);
            d3 = dot4(c3, x.a[12 + i], d3);
        }
        D[0] = d0;
        D[1] = d1;
        D[2] = d2;
        D[3] = d3;
    }
    // int8 scale of group j of this unit (group index 8h + t + 2j).
    __device__ static __forceinline__ int scale(const W& w, int u, int j) {
        const int t = u & 1;
        const int k = t + 2 * j;  // byte within sc[8h .. 8h+7]
        return k < 4 ? sbyte(w.sc.x, k) : sbyte(w.sc.y, k - 4);
    }
    // Activation element offset (within the row) of group j of unit u.
    __device__ static __forceinline__ int act_offset(int u, int j) {
        const int S = u >> 2, h = (u >> 1) & 1, t = u & 1;
        return 256 * S + 128 * h + 16 * t + 32 * j;
    }
};

// ------------------------------------------------------------------ Q4_0 --
struct Q40 {
    static constexpr int BLK_BYTES = 18;
    static constexpr int NDOT = 2;
    struct W {
        u32x4 q0, q1;
        uint32_t d0, d1;
    };
    // has1: whether block 2u+1 exists (the row may hold an odd number of
    // blocks).  A missing block re-reads block 2u (always in bounds, no
    // branch around the load) and gets d1 = 0, so its term is exactly zero.
    __device__ static __forceinline__ void load(const uint8_t* row, int u, bool has1, W& w) {
        const uint8_t* p = row + 2 * BLK_BYTES * u;
        const uint8_t* p1 = has1 ? p + BLK_BYTES : p;
        w.d0 = ld2(p);
        w.q0 = ld16(p + 2);
        const uint32_t d1 = ld2(p1);
        w.d1 = has1 ? d1 : 0u;
        w.q1 = ld16(p1 + 2);
    }
    // Block 2u is a[0..7], block 2u+1 is a[8..15]; init = -8 * s_b folds the
    // code offset into the accumulator: D = sum (code - 8) * q.
    __device__ static __forceinline__ void dots(const W& w, const Act16& x, const int init[2],
                                                int D[2]) {
        int d0 = init[0], d1 = init[1];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            d0 = dot4(w.q0[i] & LO4, x.a[i], d0);
            d0 = dot4((w.q0[i] >> 4) & LO4, x.a[4 + i], d0);
            d1 = dot4(w.q1[i] & LO4, x.a[8 + i], d1);
            d1 = dot4((w.q1[i] >> 4) & LO4, x.a[12 + i], d1);
        }
        D[0] = d0;
        D[1] = d1;
    }
};

// ------------------------------------------------------------------ Q8_0 --
struct Q80 {
    static constexpr int BLK_BYTES = 34;
    static constexpr int NDOT = 2;
    struct W {
        u32x4 a0, b0, a1, b1;
        uint32_t d0, d1;
    };
    // A missing second block re-reads block 2u and gets d1 = 0 (see Q40).
    __device__ static __forceinline__ void load(const uint8_t* row, int u, bool has1, W& w) {
        const uint8_t* p = row + 2 * BLK_BYTES * u;
        const uint8_t* p1 = has1 ? p + BLK_BYTES : p;
        w.d0 = ld2(p);
        w.a0 = ld16(p + 2);
        w.b0 = ld16(p + 18);
        const uint32_t d1 = ld2(p1);
        w.d1 = has1 ? d1 : 0u;
        w.a1 = ld16(p1 + 2);
        w.b1 = ld16(p1 + 18);
    }
    __device__ static __forceinline__ void dots(const W& w, const Act16& x, int D[2]) {
        int d0 = 0, d1 = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            d0 = dot4(w.a0[i], x.a[i], d0);
            d0 = dot4(w.b0[i], x.a[4 + i], d0);
            d1 = dot4(w.a1[i], x.a[8 + i], d1);
            d1 = dot4(w.b1[i], x.a[12 + i], d1);
        }
        D[0] = d0;
        D[1] = d1;
    }
};

// Sum of 16 activation codes (4 dwords) via dot with all-ones bytes.
__device__ __forceinline__ int sum16(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3) {
    int s = dot4(a0, 0x01010101u, 0);
    s = dot4(a1, 0x01010101u, s);
    s = dot4(a2, 0x01010101u, s);
    return dot4(a3, 0x01010101u, s);
}

}  // namespace qgemv
