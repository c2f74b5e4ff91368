// nvfp4_device.hpp -- device-side building blocks of the bf16 -> NVFP4 cast
// for gfx950 (CDNA4).  Every floating-point step is one IEEE binary32 op
// rounded to nearest-even (the library is built with -ffp-contract=off and
// fp32 denormals preserved); fused multiply-adds appear only where written.
//
// The arithmetic follows the per-token NVFP4 recipe page (TransformerEngine
// PR #3045, "Add NVFP4 per-token quantization recipe": outer amax per tensor
// or per row/column, 16-element E4M3 block scale relative to the outer scale,
// E2M1 data two per byte) with the block-scale order read from the FP8
// block-scale discussion on Model-Optimizer PR #2598:
//   S = A / 2688;  sf = (b / 6) / S;  code = E4M3(sf);  r = decode(code) * S;
//   nibble = E2M1(v / r)   (S == 0 or r == 0: code 0, sign-only nibble).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ bf16 helpers

// a 32-bit word holds two bf16 values: element 2i in the low half
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// elementwise max of two packed pairs of bf16 magnitudes (sign bits cleared
// by the caller): magnitude bit patterns order like the values they encode
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    u16x2 x = __builtin_bit_cast(u16x2, a), y = __builtin_bit_cast(u16x2, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}
__device__ __forceinline__ uint32_t abs2(uint32_t w) { return w & 0x7fff7fffu; }
__device__ __forceinline__ uint32_t max_halves(uint32_t w) {
    uint32_t lo = w & 0xffffu, hi = w >> 16;
    return lo > hi ? lo : hi;
}
// magnitude bits (16-bit) -> fp32 value
__device__ __forceinline__ float mag_to_f32(uint32_t m16) { return __uint_as_float(m16 << 16); }

// --------------------------------------------------------------- E4M3 code

// RNE onto OCP E4M3 (bias 7, 3 mantissa bits), saturating at 448 (0x7E);
// s >= 0.  Written from the format definition with integer rounding of the
// fp32 encoding; independent of the CPU reference's formulation.
__device__ __forceinline__ uint32_t e4m3_code(float s) {
    if (!(s < 448.0f)) return 0x7Eu;
    uint32_t u = __float_as_uint(s);
    if (u < 0x3C800000u) {
        // below 2^-6: code = RNE(s * 2^9), s * 2^9 < 8 exact; adding 2^23
        // leaves a unit spacing, so the addition performs the rounding
        float t = s * 512.0f + 8388608.0f;
        return __float_as_uint(t) - 0x4B000000u;
    }
    // round the 23-bit mantissa to 3 bits, ties to even; a carry moves into
    // the exponent as it should
    uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
    return (r >> 20) - 0x3C0u;  // rebias 127 -> 7 (120 << 3)
}

__device__ __forceinline__ float e4m3_value(uint32_t code) {
    // code < 8: subnormal m * 2^-9; otherwise exponent field + 120 in fp32
    return code < 8u ? (float)code * 0.001953125f : __uint_as_float((code << 20) + 0x3C000000u);
}

// ------------------------------------------------------------ block state

struct BlockScale {
    float r;        // decode(code) * S: the divisor of every element
    uint32_t code;  // E4M3 byte
    bool zero;      // r == 0: sign-only nibbles
};

// Exact block scale with IEEE divisions.  S: outer scale of the vector
// (A / 2688); bmag: block max magnitude bits (16-bit)
__device__ __forceinline__ BlockScale block_scale(uint32_t bmag, float S) {
    BlockScale bs;
    if (S == 0.0f) {
        bs.r = 0.0f; bs.code = 0u; bs.zero = true;
        return bs;
    }
    float b = mag_to_f32(bmag);
    float t = b / 6.0f;
    float sf = t / S;
    bs.code = e4m3_code(sf);
    bs.r = e4m3_value(bs.code) * S;
    bs.zero = bs.r == 0.0f;
    return bs;
}

// E2M1 of two quotients into byte SEL of `old`: gfx950's scaled FP4
// conversion with scale 1.0 rounds to nearest-even on the E2M1 grid and
// saturates at 6 (verified against the rounding table over every fp32 input);
// src0 lands in the low nibble.
template <int SEL>
__device__ __forceinline__ uint32_t put_fp4x2(uint32_t old, float q0, float q1) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, q0, q1, 1.0f, SEL);
}

// outer scale from an outer amax
__device__ __forceinline__ float outer_scale(float A) { return A / 2688.0f; }

// two fp32 values rounded to bf16 nearest-even by the hardware's packed
// conversion (checked against the integer rounding over every non-NaN fp32
// pattern): a in the low half, b in the high half
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
    const bf16x2_t p = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, p);
}

// ------------------------------------------------------------- fast path
//
// The hot loops avoid IEEE division.  Facts, each checked exhaustively (1,
// 1b and 4 on the host by tests/native/div_identity_check.c, 2 and 3 on the
// GPU):
//  1. for a bf16 numerator a and divisor r with y = RN(1/r), the sequence
//     q0 = a*y; e = fma(r, q0, -a); q = fma(-e, y, q0) returns RN(a/r)
//     (Markstein's correction) whenever r is in [2^-64, 2^64] and |a|*y <=
//     2^64, signed zeros included;
//  1b. the same sequence returns RN(t/S) for t = RN(b/6), b bf16, and any
//     normal S (t has only 128 significands, each checked against every
//     significand of S);
//  2. v_rcp_f32 returns RD(1/r) or RU(1/r) (exactly 1/r when that is
//     representable) for every normal r in [2^-64, 2^64]; one Newton step,
//     fma(fma(-r, y0, 1), y0, y0), then gives RN(1/r);
//  3. the scaled FP4 conversion rounds like the E2M1 table (put_fp4x2);
//  4. the two-op element quotient below (quot2) gives the E2M1 code of
//     RN(a/r) for bf16 a (host check, with one excluded divisor pattern).
// Blocks outside these ranges, or whose scale falls in the E4M3 subnormal
// range, take an exact slow path chosen per wave.

// RN(1/r) for normal r in [2^-64, 2^64] (fact 2)
__device__ __forceinline__ float rcp_rn(float r) {
    float y0 = __builtin_amdgcn_rcpf(r);
    float e = __builtin_fmaf(-r, y0, 1.0f);
    return __builtin_fmaf(e, y0, y0);
}

// RD(1/r) for normal r in [2^-64, 2^64]: the hardware reciprocal is RD or
// RU (fact 2); step down one ulp when the residual 1 - r*y0 is negative
__device__ __forceinline__ float rcp_rd(float r) {
    const float y0 = __builtin_amdgcn_rcpf(r);
    const float e = __builtin_fmaf(-r, y0, 1.0f);
    return __uint_as_float(__float_as_uint(y0) - (__float_as_uint(e) >> 31));
}

// RN(a / r) given y = RN(1/r), under the range conditions of fact 1
__device__ __forceinline__ float div_fast(float a, float r, float y) {
    float q0 = a * y;
    float e = __builtin_fmaf(r, q0, -a);
    return __builtin_fmaf(-e, y, q0);
}

// outer scale of one vector with its reciprocal
struct Outer {
    float S, yS;
    bool slow;   // A outside [2^-40, 2^60] (or tiny enough for S to underflow): exact path
};

// A == 0 uses S = yS = 1: when the amax was measured on the vector, every
// block of it is all zeros and the fast block below encodes it as code 0
// with sign-only nibbles.  SAT: the amax comes from the caller and may be 0
// over nonzero data, where S == 0 must still give code 0 and sign-only
// nibbles; such a vector (valid: it lies inside the tensor) takes the exact
// path, whose block scale handles S == 0.
template <bool SAT = false>
__device__ __forceinline__ Outer make_outer(float A, bool valid = true) {
    Outer o;
    const bool zero = A == 0.0f;
    o.S = zero ? 1.0f : outer_scale(A);
    o.yS = rcp_rn(o.S);
    o.slow = zero ? (SAT && valid) : !(A >= 0x1p-40f && A <= 0x1p60f);
    return o;
}

// Outer scale of a vector as kept in LDS: S and 1/S, the reciprocal negated
// when the vector needs the exact path (an amax outside the fast range)
__device__ __forceinline__ float2 outer_entry(float A) {
    const Outer o = make_outer(A);
    return make_float2(o.S, o.slow ? -o.yS : o.yS);
}

__device__ __forceinline__ Outer outer_from(float2 e) {
    Outer o;
    o.S = e.x;
    o.yS = __builtin_fabsf(e.y);
    o.slow = e.y < 0.0f;
    return o;
}

// Per-block parameters on the fast path: the split reciprocal yh = RD(1/r),
// yl = RN((1 - r*yh) * yh) >= 0 of the divisor r = decode(code) * S, used
// by the two-op element quotient, and the E4M3 scale byte in the low 8 bits
// of `code` (the bits above are ignored by byte stores).  slow: this block
// needs the exact path.  The outer scale's own range flag is not included.
struct FastBlock {
    float yh, yl;
    uint32_t code;
    bool slow;
};

// Element quotient for the E2M1 code: fma(a, yh, a*yl).  Its E2M1 code
// equals that of RN(a/r) for every bf16 a and every r in the fast range
// except r with all mantissa bits set (fact 4, checked exhaustively on the
// host; fast_block sends those blocks to the exact path).  yl >= 0 keeps the
// sign of a zero numerator.
__device__ __forceinline__ float quot2(float a, float yh, float yl) {
    return __builtin_fmaf(a, yh, a * yl);
}

constexpr float kRcp6 = 0x1.555556p-3f;   // RN(1/6)

// bbits: the block's largest magnitude as fp32 bits (a bf16 magnitude in the
// high half, zeros below).  SAT: the outer amax may be smaller than the data
// (caller-supplied amax), so the block scale may saturate and quotients
// exceed 6.  SUB: blocks with a scale in the E4M3 subnormal range stay on
// the fast path (below); without it they go to the exact path, which costs
// the kernels that rarely meet them nothing on their common path.
template <bool SAT, bool SUB = false>
__device__ __forceinline__ FastBlock fast_block(uint32_t bbits, const Outer& o) {
    FastBlock fb;
    const float b = __uint_as_float(bbits);
    const float t = div_fast(b, 6.0f, kRcp6);   // RN(b / 6)   (fact 1: b is bf16)
    const float sf = div_fast(t, o.S, o.yS);    // RN(t / S)   (fact 1b: t = RN(b/6))
    const uint32_t u = __float_as_uint(sf);
    // E4M3 code of sf by rounding its fp32 encoding: mantissa to 3 bits, ties
    // to even (a carry moves into the exponent).  c holds the fp32 exponent
    // and the 3 kept mantissa bits plus 0x40, so that its low byte is the
    // E4M3 code (the bias change 127 -> 7 is 120 << 3 = 0x3C0 = 0x400 - 0x40).
    // The clamp to [0x400, 0x47E] gives code 0 for an all-zero block (its
    // elements are +/-0, so the divisor's value does not matter) and
    // saturates at 448 (0x7E).
    uint32_t c = (u + (0x7FFFFu + (0x40u << 20)) + ((u >> 20) & 1u)) >> 20;
    c = c < 0x400u ? 0x400u : (c > 0x47Eu ? 0x47Eu : c);
    fb.code = c;
    float r = __uint_as_float((c << 20) - (0x40u << 20)) * o.S;   // decode(code) * S; 2^-7 * S for code 0
    fb.yh = rcp_rd(r);
    fb.yl = __builtin_fmaf(-r, fb.yh, 1.0f) * fb.yh;
    // 0 < sf < 2^-6 (rare: a block far below its vector's amax) is the E4M3
    // subnormal range: code = RNE(sf * 2^9) in 0..8 (8 is 2^-6, the smallest
    // normal; sf * 2^9 < 8 is exact and adding 2^23 leaves a unit spacing,
    // so the addition rounds), r = code * 2^-9 * S.  Code 0 (sf < 2^-10) has
    // r = 0: yh = yl = 0 make every quotient a zero of the element's sign,
    // the sign-only nibbles the definition gives.  Taken by the whole wave
    // when any lane needs it (a uniform branch costs the common case less
    // than a divergent one).
    const bool sub = (u - 1u) < (0x3C800000u - 1u);
    if (SUB && __builtin_amdgcn_ballot_w64(sub) != 0ull) {
        const uint32_t m = __float_as_uint(sf * 512.0f + 8388608.0f) - 0x4B000000u;
        const float rs = ((float)m * 0x1p-9f) * o.S;
        const float yhs = m == 0u ? 0.0f : rcp_rd(rs);
        const float yls = __builtin_fmaf(-rs, yhs, 1.0f) * yhs;
        fb.code = sub ? m : fb.code;
        r = sub ? rs : r;
        fb.yh = sub ? yhs : fb.yh;
        fb.yl = sub ? yls : fb.yl;
    }
    // exact path: an r with all mantissa bits set (fact 4's exception), and
    // without SUB a scale in the E4M3 subnormal range
    bool slow = (!SUB && sub) || (__float_as_uint(r) & 0x7FFFFFu) == 0x7FFFFFu;
    if (SAT) slow |= !(r <= 0x1p64f && b * fb.yh <= 0x1p64f);
    fb.slow = slow;
    return fb;
}

// ------------------------------------------------ buffers and lane exchange

// Buffer resources: a raw buffer over [base, base + bytes) (bytes <= 2^31).
// Loads at an offset at or beyond `bytes` read zeros and stores there are
// dropped, which is how rows past the end of the tensor and lanes past its
// last column are handled.  The offset checked is the lane offset plus the
// scalar offset (checked on gfx950 with an in-bounds probe), so the per-row
// part of an address goes in the scalar offset at no vector-ALU cost; sums
// stay below 2^32.  The fourth descriptor word is the raw-buffer setting of
// the gfx9 family.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kCacheNT = 2;               // nontemporal hint in the gfx940-family cache-policy bits
constexpr uint32_t kOffOut = 0x80000000u; // lane offset beyond every buffer's extent

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// DPP: value of the neighbouring lane (lane ^ 1)
__device__ __forceinline__ uint32_t from_pair(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t rowmax_word(const u32x4& w) {
    return pk_max_u16(pk_max_u16(abs2(w.x), abs2(w.y)), pk_max_u16(abs2(w.z), abs2(w.w)));
}

// DPP quad permutations: the value of the even / odd lane of each pair
__device__ __forceinline__ float from_even(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xA0, 0xF, 0xF, false));   // [0,0,2,2]
}
__device__ __forceinline__ float from_odd(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xF5, 0xF, 0xF, false));   // [1,1,3,3]
}

// ----------------------------------------------------------- grouped table

// Experts for the grouped cast travel in the kernel arguments: row offsets
// (multiples of 16) and counts.
constexpr int kMaxGroupsPerLaunch = 128;
struct GroupTable {
    int32_t n;
    int32_t first;                        // index of table entry 0 among all experts
    int64_t off[kMaxGroupsPerLaunch];     // first row of each expert
    int64_t cnt[kMaxGroupsPerLaunch];     // rows of each expert
};

// expert owning row r, moving forward from entry g (an entry whose offset
// is <= r): rows only grow within a workgroup's walk, so this is usually no
// step at all, where a fresh search costs a chain of dependent table loads
__device__ __forceinline__ int group_advance(const GroupTable& gt, int g, int64_t r) {
    while (g + 1 < gt.n && gt.off[g + 1] <= r) ++g;
    return g;
}

// expert owning row r (r inside the table's span): the last entry whose
// offset is <= r, which skips empty experts sharing that offset
__device__ __forceinline__ int group_of_row(const GroupTable& gt, int64_t r) {
    int lo = 0, hi = gt.n - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (gt.off[mid] <= r) lo = mid; else hi = mid - 1;
    }
    return lo;
}

}  // namespace nvfp4
