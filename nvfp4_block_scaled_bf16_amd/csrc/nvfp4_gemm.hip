// nvfp4_gemm.hip -- the NVFP4 GEMM consumer for gfx950: two NVFP4 operands
// with 16-element blocks along the contraction dimension K, rescaled by the
// per-row / per-column outer scales in the epilogue (the GEMM of the per-token
// recipe page, TransformerEngine PR #3045, "Changes" and the sequence
// diagram's TN forward product; its NN dgrad and NT wgrad products are this
// form applied to the cast's columnwise output):
//   out[m][n] = S_a(m) * S_b(n) * sum_k (g * D)_a[m][k] * (g * D)_b[n][k]
// with g the E2M1 value, D the decoded E4M3 block scale and S = amax / 2688.
//
// g * D has at most 6 significant bits and lies in [2^-10, 2688], so it is
// exact in fp16: each K step dequantizes the operands' FP4 bytes (hardware
// FP4 -> fp16 conversion, then one packed fp16 multiply by D per pair) into
// fp16 tiles in LDS, and the contraction runs on fp16 MFMA
// (v_mfma_f32_32x32x16_f16, same rate as bf16) with fp32 accumulation; the
// outer scales multiply the accumulators in the epilogue.  (gfx950's scaled
// FP4 MFMA takes one power-of-two scale per 32 elements and cannot carry an
// E4M3 scale per 16; E4M3 * E2M1 products need up to 6 significant bits, more
// than any 8-bit format holds.)
//
// Every output element sees the same sequence of MFMAs (K in 16-wide chunks,
// in order) whatever the tile shape, so the result does not depend on the
// tile configuration chosen.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "nvfp4_device.hpp"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kStepK = 64;                  // K per pipeline step: 4 scale blocks
constexpr int kPitch = kStepK + 8;          // fp16 per LDS tile row (padding spreads the rows over the banks)

// E4M3 code -> value (exact): the code's bits placed in an fp32 exponent and
// mantissa field are the value times 2^-120 (subnormal codes become fp32
// subnormals, which this code keeps)
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) { return __uint_as_float(code << 20) * 0x1p120f; }

// buffer descriptor over `bytes` bytes at base; loads at offsets past the end
// return zeros
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOob = 0x80000000u;   // an offset past every descriptor's end

// One thread's share of a K step for one operand: 32 consecutive elements
// (two scale blocks) of one row.  Rows past the end and blocks past K read
// as zeros.
struct RowPiece {
    uint32_t q[4];      // 16 bytes: 32 nibbles, element 2i in the low nibble
    uint32_t sf;        // two scale codes: low byte, next byte (0 where the
                        // scales come in 16-byte groups instead)
};

// Byte offset of scale block c of row `row` (both within the operand tile,
// whose first row is a multiple of 128).  Plain: row-major [rows][K/16].
// Swizzled (SWZ): the GEMM layout of 128-row x 4-block tiles of 512 bytes,
// row-tile major, row r in 16-byte line r % 32 at 4-byte slot (r / 32) % 4,
// block c at byte c % 4; nbp = K/16 rounded up to 4.  Blocks c and c + 1 (c
// even) are adjacent in both.
template <bool SWZ>
__device__ __forceinline__ uint32_t scale_offset(uint32_t row, uint32_t c, uint32_t K) {
    if (!SWZ) return row * (K / 16) + c;
    const uint32_t nbp = (K / 16 + 3) & ~3u;
    return (row >> 7) * (128u * nbp) + (c >> 2) * 512u + (row & 31u) * 16u + ((row >> 5) & 3u) * 4u + (c & 3u);
}

// row: the row within the operand tile (descriptors q_rs / s_rs start at the
// tile's first row and end after its last valid row, for swizzled scales
// after its last 128-row group); k0 % 32 == 0.  A64 (K % 64 == 0): every
// K step is whole, so a piece is one 16-byte load of codes (16-byte
// aligned) and one 4-byte load holding its two scale bytes (the step's four
// blocks sit in one aligned word, plain or swizzled); else two 8-byte loads
// and two byte loads, each guarded against K.
template <bool SWZ, bool A64>
__device__ __forceinline__ RowPiece load_piece(__amdgpu_buffer_rsrc_t q_rs, __amdgpu_buffer_rsrc_t s_rs, uint32_t row,
                                               uint32_t K, uint32_t k0) {
    const uint32_t off = row * (K / 2) + k0 / 2, soff = scale_offset<SWZ>(row, k0 / 16, K);
    const bool lo_ok = k0 < K, hi_ok = k0 + 16 < K;
    if (A64) {
        const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(q_rs, lo_ok ? off : kOob, 0, 0);
        const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(s_rs, lo_ok ? (soff & ~3u) : kOob, 0, 0);
        return RowPiece{{q.x, q.y, q.z, q.w}, (w >> (8 * (soff & 3u))) & 0xffffu};
    }
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 lo = __builtin_amdgcn_raw_buffer_load_b64(q_rs, lo_ok ? off : kOob, 0, 0);
    const u32x2 hi = __builtin_amdgcn_raw_buffer_load_b64(q_rs, hi_ok ? off + 8 : kOob, 0, 0);
    const uint32_t s0 = __builtin_amdgcn_raw_buffer_load_b8(s_rs, lo_ok ? soff : kOob, 0, 0);
    const uint32_t s1 = __builtin_amdgcn_raw_buffer_load_b8(s_rs, hi_ok ? soff + 1 : kOob, 0, 0);
    return RowPiece{{lo.x, lo.y, hi.x, hi.y}, s0 | (s1 << 8)};
}

// dequantize a piece (its codes, and the two scale codes in sf) into 32
// fp16 (g * D, exact) and store them to LDS
__device__ __forceinline__ void store_piece(const RowPiece& p, uint32_t sf, _Float16* dst) {
    const _Float16 d0 = (_Float16)e4m3_to_f32(sf & 0xffu), d1 = (_Float16)e4m3_to_f32(sf >> 8);
    f16x8 out[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const f16x2 d = w < 2 ? f16x2{d0, d0} : f16x2{d1, d1};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            // byte b of word w: elements 8w + 2b (low nibble) and 8w + 2b + 1;
            // the conversion with scale 1.0 gives the E2M1 values exactly and
            // the packed product with D is exact in fp16
            f16x2 g;
            if (b == 0) g = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(p.q[w], 1.0f, 0);
            else if (b == 1) g = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(p.q[w], 1.0f, 1);
            else if (b == 2) g = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(p.q[w], 1.0f, 2);
            else g = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(p.q[w], 1.0f, 3);
            const f16x2 v = g * d;
            out[w][2 * b] = v.x;
            out[w][2 * b + 1] = v.y;
        }
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) *reinterpret_cast<f16x8*>(dst + 8 * w) = out[w];
}

// One workgroup computes a TM x TN output tile with WM x WN waves, each wave
// a (TM / WM) x (TN / WN) block of 32 x 32 MFMA tiles.  LDS holds the tile's
// TM rows of A then TN rows of B, kStepK fp16 values each, double buffered.
// Each K step a row is loaded as two 32-element pieces; piece p (p = t + NT i
// for thread t, i < P) is row p / 2, half p % 2, so each i is all-A or all-B.
template <int TM, int TN>
using GemmLds = _Float16[2][(TM + TN) * kPitch];

// XCD-aware order over a one-dimensional grid: each of the 8 XCDs (own L2)
// takes a contiguous run of tile indices (band_order maps an index to a tile),
// so the operand rows those tiles share are reused from one L2
__device__ __forceinline__ uint32_t xcd_tile() {
    const uint32_t ntiles = gridDim.x, lin = blockIdx.x;
    return (ntiles & 7u) == 0u ? (lin & 7u) * (ntiles >> 3) + (lin >> 3) : lin;
}

// Tile t of an ntm x ntn grid in groups of kBandGroup row bands: within a
// group, down the bands of one column of tiles, then the next column.  Runs
// of consecutive tiles (as one XCD holds them at a time) thus share a few
// row bands of A and a few column tiles of B instead of one band of A and
// every tile of B, so fewer distinct operand rows stream through its L2 per
// K step.
constexpr uint32_t kBandGroup = 4;
__device__ __forceinline__ void band_order(uint32_t t, uint32_t ntm, uint32_t ntn, uint32_t* by, uint32_t* bx) {
    const uint32_t per = kBandGroup * ntn, g = t / per, first = g * kBandGroup;
    const uint32_t gm = ntm - first < kBandGroup ? ntm - first : kBandGroup, w = t - g * per;
    *by = first + w % gm;
    *bx = w / gm;
}

// the output tile at (m0, n0) of out [M][N] = A [M][K] x B [N][K]^T
template <int TM, int TN, int WM, int WN, bool SWZ, bool A64>
__device__ __forceinline__ void gemm_tile(const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_sf,
                                          const float* __restrict__ a_amax, int a_per_row,
                                          const uint8_t* __restrict__ b_q, const uint8_t* __restrict__ b_sf,
                                          const float* __restrict__ b_amax, int b_per_row, int64_t M, int64_t N,
                                          int64_t K, int64_t m0, int64_t n0, float* __restrict__ out,
                                          GemmLds<TM, TN>& S) {
    constexpr int NT = 64 * WM * WN, ROWS = TM + TN, P = 2 * ROWS / NT;
    constexpr int FM = TM / WM / 32, FN = TN / WN / 32;
    static_assert(2 * ROWS % NT == 0 && 2 * TM % NT == 0 && FM >= 1 && FN >= 1, "tile shape");
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave / WN, wn = wave % WN;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    // descriptors over the tile's valid rows of each operand
    const uint32_t va = (uint32_t)(M - m0 < TM ? M - m0 : TM), vb = (uint32_t)(N - n0 < TN ? N - n0 : TN);
    const uint32_t Ku = (uint32_t)K;
    const __amdgpu_buffer_rsrc_t aq_rs = gemm_rsrc(a_q + m0 * (K / 2), va * (Ku / 2));
    const __amdgpu_buffer_rsrc_t bq_rs = gemm_rsrc(b_q + n0 * (K / 2), vb * (Ku / 2));
    // swizzled scales: the tile's whole 128-row groups (their padding bytes
    // multiply rows that read as zeros)
    const uint32_t nbp = (Ku / 16 + 3) & ~3u;
    const __amdgpu_buffer_rsrc_t as_rs =
        SWZ ? gemm_rsrc(a_sf + m0 * nbp, ((va + 127u) & ~127u) * nbp) : gemm_rsrc(a_sf + m0 * (K / 16), va * (Ku / 16));
    const __amdgpu_buffer_rsrc_t bs_rs =
        SWZ ? gemm_rsrc(b_sf + n0 * nbp, ((vb + 127u) & ~127u) * nbp) : gemm_rsrc(b_sf + n0 * (K / 16), vb * (Ku / 16));

    // two register sets for the raw bytes of the next two K steps
    RowPiece pc[P], pn[P];
    // SG (plain scale layout, K % 64 == 0): a piece's scale bytes come from
    // one 16-byte load per four K steps (the row's blocks 16 g .. 16 g + 15
    // for steps 4 g .. 4 g + 3; dword-aligned as K / 16 % 4 == 0), issued
    // with the codes of step 4 g into sg_nxt and moved to sg_cur when step
    // 4 g is dequantized, instead of one 4-byte load per step: a quarter of
    // the scale loads, each of which touches one cache line per row.  Bytes
    // read past a row's last block belong to steps past K and are masked.
    constexpr bool SG = A64 && !SWZ;
    u32x4 sg_cur[SG ? P : 1], sg_nxt[SG ? P : 1];
    // kbase = 64 s for step s; J = s % 4
    auto load_all = [&](RowPiece* dst, uint32_t kbase, auto J) {
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int p = t + NT * i, r = p >> 1;
            const uint32_t k0 = kbase + 32 * (p & 1);
            const bool is_a = (NT * i) / 2 < TM;
            const uint32_t row = (uint32_t)(is_a ? r : r - TM);
            if (SG) {
                const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(is_a ? aq_rs : bq_rs,
                                                                      k0 < Ku ? row * (Ku / 2) + k0 / 2 : kOob, 0, 0);
                dst[i] = RowPiece{{q.x, q.y, q.z, q.w}, 0u};
                if (decltype(J)::value == 0)
                    sg_nxt[i] = __builtin_amdgcn_raw_buffer_load_b128(
                        is_a ? as_rs : bs_rs, kbase < Ku ? row * (Ku / 16) + kbase / 16 : kOob, 0, 0);
            } else {
                dst[i] = load_piece<SWZ, A64>(is_a ? aq_rs : bq_rs, is_a ? as_rs : bs_rs, row, Ku, k0);
            }
        }
    };
    auto store_all = [&](const RowPiece* src, int buf, uint32_t kbase, auto J) {
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int p = t + NT * i;
            uint32_t sf = src[i].sf;
            if (SG) {
                constexpr int w = decltype(J)::value;
                if (w == 0) sg_cur[i] = sg_nxt[i];
                sf = kbase < Ku ? (sg_cur[i][w] >> (16 * (p & 1))) & 0xffffu : 0u;
            }
            store_piece(src[i], sf, &S[buf][(p >> 1) * kPitch + 32 * (p & 1)]);
        }
    };
    using J0 = std::integral_constant<int, 0>;
    using J1 = std::integral_constant<int, 1>;
    using J2 = std::integral_constant<int, 2>;
    using J3 = std::integral_constant<int, 3>;

    const uint32_t nk = (Ku + kStepK - 1) / kStepK;
    // One K step: load the bytes of step kt + 2 into `nxt` (zeros past K),
    // run step kt's MFMAs from its LDS buffer, dequantize step kt + 1's bytes
    // (`cur`, loaded a step earlier) into the other buffer.  Steps alternate
    // the two register sets, so a load stays in flight through a whole step
    // (copying one set into the other would wait for it).  The buffer written
    // in the last step is never read.
    // JN = (kt + 2) % 4, JC = (kt + 1) % 4
    auto step = [&](uint32_t kt, RowPiece* cur, RowPiece* nxt, auto JN, auto JC) {
        const int buf = (int)(kt & 1);
        // the compiler's single-wave MFMA interleave for this block: spreads
        // the LDS reads and the dequantization between the MFMAs (measured
        // 4-5 % faster than its default schedule)
        __builtin_amdgcn_iglp_opt(1);
        load_all(nxt, (kt + 2) * kStepK, JN);
        const _Float16* as = S[buf] + (wm * (TM / WM)) * kPitch;
        const _Float16* bs = S[buf] + (TM + wn * (TN / WN)) * kPitch;
#pragma unroll
        for (int kc = 0; kc < kStepK / 16; ++kc) {
            const int kk = 16 * kc + 8 * (lane >> 5);
            f16x8 fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[i] = *reinterpret_cast<const f16x8*>(as + (32 * i + (lane & 31)) * kPitch + kk);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                fb[j] = *reinterpret_cast<const f16x8*>(bs + (32 * j + (lane & 31)) * kPitch + kk);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        store_all(cur, buf ^ 1, (kt + 1) * kStepK, JC);
        __syncthreads();
    };
    load_all(pc, 0, J0{});
    store_all(pc, 0, 0, J0{});
    load_all(pc, kStepK, J1{});
    __syncthreads();
    if constexpr (SG) {
        for (uint32_t kt = 0; kt < nk; kt += 4) {
            step(kt, pc, pn, J2{}, J1{});
            if (kt + 1 < nk) step(kt + 1, pn, pc, J3{}, J2{});
            if (kt + 2 < nk) step(kt + 2, pc, pn, J0{}, J3{});
            if (kt + 3 < nk) step(kt + 3, pn, pc, J1{}, J0{});
        }
    } else {   // the step index modulo 4 is not used: unrolled twice (measured faster here)
        for (uint32_t kt = 0; kt < nk; kt += 2) {
            step(kt, pc, pn, J0{}, J0{});
            if (kt + 1 < nk) step(kt + 1, pn, pc, J0{}, J0{});
        }
    }

    // epilogue: out = RN(RN(acc * S_a) * S_b); accumulator a of lane l holds
    // row 8 (a / 4) + 4 (l / 32) + a % 4, column l % 32 of its 32 x 32 block
    const float sa_t = a_per_row ? 0.0f : outer_scale(a_amax[0]);
    const float sb_t = b_per_row ? 0.0f : outer_scale(b_amax[0]);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int64_t col = n0 + wn * (TN / WN) + 32 * j + (lane & 31);
        const bool col_ok = col < N;
        const float sb = b_per_row ? (col_ok ? outer_scale(b_amax[col]) : 0.0f) : sb_t;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int a = 0; a < 16; ++a) {
                const int64_t row = m0 + wm * (TM / WM) + 32 * i + 8 * (a >> 2) + 4 * (lane >> 5) + (a & 3);
                if (row < M && col_ok) {
                    const float sa = a_per_row ? outer_scale(a_amax[row]) : sa_t;
                    out[row * N + col] = (acc[i][j][a] * sa) * sb;
                }
            }
        }
    }
}

// Grid: cdiv(M, TM) * cdiv(N, TN) workgroups (one dimension); ntn = cdiv(N, TN).
// SWZ: both operands' scales in the swizzled layout; A64: K % 64 == 0.
template <int TM, int TN, int WM, int WN, bool SWZ, bool A64>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm_nvfp4(
    const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_sf, const float* __restrict__ a_amax,
    int a_per_row, const uint8_t* __restrict__ b_q, const uint8_t* __restrict__ b_sf,
    const float* __restrict__ b_amax, int b_per_row, int64_t M, int64_t N, int64_t K, uint32_t ntn,
    float* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) GemmLds<TM, TN> S;
    uint32_t by, bx;
    band_order(xcd_tile(), gridDim.x / ntn, ntn, &by, &bx);
    gemm_tile<TM, TN, WM, WN, SWZ, A64>(a_q, a_sf, a_amax, a_per_row, b_q, b_sf, b_amax, b_per_row, M, N, K,
                                        (int64_t)by * TM, (int64_t)bx * TN, out, S);
}

// Grouped: group g (the table's entry g, expert first + g) multiplies A's
// rows off[g] .. off[g] + cnt[g] by its own B (expert first + g of b_*),
// writing out's same rows.  Tiles of group g are tstart[g] .. tstart[g + 1];
// grid: tstart[n] workgroups.
template <int TM, int TN, int WM, int WN, bool A64>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm_nvfp4_grouped(
    const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_sf, const float* __restrict__ a_amax,
    int a_per_row, const uint8_t* __restrict__ b_q, const uint8_t* __restrict__ b_sf,
    const float* __restrict__ b_amax, int b_per_row, GemmGroups gg, int64_t N, int64_t K, uint32_t ntn,
    float* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) GemmLds<TM, TN> S;
    const uint32_t tile = xcd_tile();
    // the last entry starting at or before this tile (skips empty groups,
    // which share the next group's start)
    int lo = 0, hi = gg.n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (gg.tstart[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    const uint32_t local = tile - gg.tstart[lo];
    const int64_t off = gg.off[lo], e = (int64_t)gg.first + lo;
    uint32_t by, bx;
    band_order(local, (uint32_t)((gg.cnt[lo] + TM - 1) / TM), ntn, &by, &bx);
    gemm_tile<TM, TN, WM, WN, false, A64>(a_q + off * (K / 2), a_sf + off * (K / 16), a_amax + (a_per_row ? off : 0), a_per_row,
                              b_q + e * N * (K / 2), b_sf + e * N * (K / 16), b_amax + (b_per_row ? e * N : e),
                              b_per_row, gg.cnt[lo], N, K, (int64_t)by * TM, (int64_t)bx * TN, out + off * N, S);
}

template <int TM, int TN, int WM, int WN, bool SWZ, bool A64>
hipError_t launch_cfg(const uint8_t* a_q, const uint8_t* a_sf, const float* a_amax, int a_per_row,
                      const uint8_t* b_q, const uint8_t* b_sf, const float* b_amax, int b_per_row, int64_t M,
                      int64_t N, int64_t K, float* out, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    const int64_t ntn = (N + TN - 1) / TN, ntiles = ntn * ((M + TM - 1) / TM);
    if (ntiles > kMaxGemmTiles) return hipErrorInvalidValue;
    hipExtLaunchKernelGGL(k_gemm_nvfp4<TM, TN, WM, WN, SWZ, A64>, dim3((unsigned)ntiles), dim3(64 * WM * WN), 0, st, ev0, ev1,
                          0, a_q, a_sf, a_amax, a_per_row, b_q, b_sf, b_amax, b_per_row, M, N, K, (uint32_t)ntn, out);
    return hipGetLastError();
}

bool sf_aligned(const uint8_t* a_sf, const uint8_t* b_sf) {
    return ((reinterpret_cast<uintptr_t>(a_sf) | reinterpret_cast<uintptr_t>(b_sf)) & 3u) == 0;
}

}  // namespace

namespace {

// Scales [R][nb] -> the swizzled layout (see scale_offset): one thread per
// output dword, which holds the four blocks 4 cb .. 4 cb + 3 of one row;
// bytes for rows >= R or blocks >= nb are zero.  Grid-stride over ndw dwords.
__global__ __launch_bounds__(256) void k_swizzle_scales(const uint8_t* __restrict__ sf, int64_t R, int64_t nb,
                                                        uint32_t* __restrict__ out, int64_t ndw) {
    const int64_t nbq = (nb + 3) / 4;
    for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < ndw; d += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = d / 128, w = d % 128;
        const int64_t r = (t / nbq) * 128 + (w & 3) * 32 + (w >> 2), c0 = (t % nbq) * 4;
        uint32_t v = 0u;
        if (r < R) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (c0 + j < nb) v |= (uint32_t)sf[r * nb + c0 + j] << (8 * j);
        }
        out[d] = v;
    }
}

}  // namespace

hipError_t launch_swizzle_scales(const uint8_t* sf, int64_t R, int64_t nb, uint8_t* out, hipStream_t st) {
    const int64_t ndw = ((R + 127) / 128 * 128) * ((nb + 3) / 4 * 4) / 4;
    if (ndw <= 0) return hipSuccess;
    int64_t grid = (ndw + 255) / 256;
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL(k_swizzle_scales, dim3((unsigned)grid), dim3(256), 0, st, sf, R, nb,
                       reinterpret_cast<uint32_t*>(out), ndw);
    return hipGetLastError();
}

hipError_t launch_gemm_nvfp4(const uint8_t* a_q, const uint8_t* a_sf, const float* a_amax, int a_per_row,
                             const uint8_t* b_q, const uint8_t* b_sf, const float* b_amax, int b_per_row,
                             int64_t M, int64_t N, int64_t K, float* out, hipStream_t st, hipEvent_t ev0,
                             hipEvent_t ev1, bool swizzled) {
    if (M <= 0 || N <= 0) return hipSuccess;
    // 256 x 256 tiles (8 waves of 128 x 64) once they fill the 256 CUs, else
    // 128 x 128 tiles (4 waves of 64 x 64) for four times the workgroups
    const bool big = ((M + 255) / 256) * ((N + 255) / 256) >= 256;
    // the wide loads also need 4-byte aligned plain scales (swizzled ones are
    // required to be); byte-aligned plain scales take the byte loads
    const bool a64 = K % 64 == 0 && (swizzled || sf_aligned(a_sf, b_sf));
#define NVFP4_GEMM_LAUNCH(TM, TN, WM, WN, SW)                                                                      \
    return a64 ? launch_cfg<TM, TN, WM, WN, SW, true>(a_q, a_sf, a_amax, a_per_row, b_q, b_sf, b_amax, b_per_row, M, \
                                                      N, K, out, st, ev0, ev1)                                     \
               : launch_cfg<TM, TN, WM, WN, SW, false>(a_q, a_sf, a_amax, a_per_row, b_q, b_sf, b_amax, b_per_row, M, \
                                                       N, K, out, st, ev0, ev1)
    if (swizzled) {
        if (big) NVFP4_GEMM_LAUNCH(256, 256, 2, 4, true);
        NVFP4_GEMM_LAUNCH(128, 128, 2, 2, true);
    }
    if (big) NVFP4_GEMM_LAUNCH(256, 256, 2, 4, false);
    NVFP4_GEMM_LAUNCH(128, 128, 2, 2, false);
#undef NVFP4_GEMM_LAUNCH
}

namespace {

template <int TM, int TN, int WM, int WN, bool A64>
hipError_t launch_grouped_cfg(const uint8_t* a_q, const uint8_t* a_sf, const float* a_amax, int a_per_row,
                              const uint8_t* b_q, const uint8_t* b_sf, const float* b_amax, int b_per_row,
                              int32_t num_groups, const int64_t* h_counts, int64_t N, int64_t K, float* out,
                              hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    const int64_t ntn = (N + TN - 1) / TN;
    // the launches that have tiles, so the trace events bracket the first and last
    int last = -1;
    for (int32_t e0 = 0; e0 < num_groups; e0 += kMaxGemmGroups)
        for (int32_t e = e0; e < num_groups && e < e0 + kMaxGemmGroups; ++e)
            if (h_counts[e] > 0) last = e0;
    int64_t off = 0;
    bool first_launch = true;
    for (int32_t e0 = 0; e0 < num_groups; e0 += kMaxGemmGroups) {
        GemmGroups gg;
        gg.n = 0;
        gg.first = e0;
        int64_t tiles = 0;
        for (int32_t e = e0; e < num_groups && e < e0 + kMaxGemmGroups; ++e) {
            gg.off[gg.n] = off;
            gg.cnt[gg.n] = h_counts[e];
            gg.tstart[gg.n] = (uint32_t)tiles;
            tiles += ntn * ((h_counts[e] + TM - 1) / TM);
            off += h_counts[e];
            ++gg.n;
        }
        gg.tstart[gg.n] = (uint32_t)tiles;
        if (tiles == 0) continue;
        if (tiles > kMaxGemmTiles) return hipErrorInvalidValue;
        hipExtLaunchKernelGGL(k_gemm_nvfp4_grouped<TM, TN, WM, WN, A64>, dim3((unsigned)tiles), dim3(64 * WM * WN), 0, st,
                              first_launch ? ev0 : nullptr, e0 == last ? ev1 : nullptr, 0, a_q, a_sf, a_amax,
                              a_per_row, b_q, b_sf, b_amax, b_per_row, gg, N, K, (uint32_t)ntn, out);
        first_launch = false;
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_gemm_grouped(const uint8_t* a_q, const uint8_t* a_sf, const float* a_amax, int a_per_row,
                               const uint8_t* b_q, const uint8_t* b_sf, const float* b_amax, int b_per_row,
                               int32_t num_groups, const int64_t* h_counts, int64_t N, int64_t K, float* out,
                               hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    if (N <= 0) return hipSuccess;
    // 256 x 256 tiles when they fill the CUs and each group's row padding to
    // 256 wastes at most a fifth of the rows
    int64_t T = 0, padded = 0, tiles256 = 0;
    for (int32_t e = 0; e < num_groups; ++e) {
        T += h_counts[e];
        padded += (h_counts[e] + 255) / 256 * 256;
        tiles256 += (h_counts[e] + 255) / 256 * ((N + 255) / 256);
    }
    const bool big = tiles256 >= 256 && 4 * padded <= 5 * T, a64 = K % 64 == 0 && sf_aligned(a_sf, b_sf);
#define NVFP4_GROUPED_LAUNCH(TM, TN, WM, WN)                                                                        \
    return a64 ? launch_grouped_cfg<TM, TN, WM, WN, true>(a_q, a_sf, a_amax, a_per_row, b_q, b_sf, b_amax,          \
                                                          b_per_row, num_groups, h_counts, N, K, out, st, ev0, ev1) \
               : launch_grouped_cfg<TM, TN, WM, WN, false>(a_q, a_sf, a_amax, a_per_row, b_q, b_sf, b_amax,         \
                                                           b_per_row, num_groups, h_counts, N, K, out, st, ev0, ev1)
    if (big) NVFP4_GROUPED_LAUNCH(256, 256, 2, 4);
    NVFP4_GROUPED_LAUNCH(128, 128, 2, 2);
#undef NVFP4_GROUPED_LAUNCH
}

}  // namespace nvfp4
