// nvfp4_rht.hip -- the cast's opt-in random Hadamard transform on the
// columnwise direction, for gfx950 (the per-token recipe page,
// TransformerEngine PR #3045, "Changes": per_token_rht, columnwise only).
//
// Each 16-element block of a columnwise vector (16 consecutive rows of one
// column of x) is replaced by y = H16 D x / 4 before the columnwise cast:
// H16 the Sylvester Hadamard matrix, D the signs of a 16-bit mask (bit i set:
// row i of the block negated).  The transform runs as the fast Walsh-Hadamard
// butterfly in binary32 (stages 1, 2, 4, 8; each pair (a, b) becomes
// (a + b, a - b)), is scaled by 1/4 and rounded to bf16, nearest-even; the
// bf16 result is cast exactly like any columnwise input, with its own amax
// (per column, or one for the tensor).
//
// Two passes over x, like the ordinary per-token cast: the amaxes (of the
// transformed columns, and of x's rows when rowwise output is wanted), then
// the transform again with both encodings (rowwise of x, columnwise of y).
// A lane holds a 16-row x 8-column sub-block (one 16-byte word per row); a
// workgroup of 4 waves covers 128 rows x 256 columns; a rowwise block is a
// lane pair.  Requires M % 16 == 0 and K % 8 == 0 (K % 16 == 0 with rowwise
// output).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_device.hpp"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

constexpr int kRhtCols = 256;        // columns per workgroup (32 lanes x 8)
constexpr int kRhtRows = 128;        // rows per workgroup step (4 waves x 2 row groups x 16)
constexpr int kRhtStagePitch = 72;   // LDS bytes per staged column: 64 (128 rows of codes) + 8 padding
constexpr int kRhtAmaxSteps = 2;     // steps per workgroup in the amax pass (256 rows: two full rounds of workgroups)

// column k (0..7) of a lane's 8-column row word, as fp32 bits
__device__ __forceinline__ uint32_t col_bits(const u32x4& w, int k) {
    const uint32_t word = (k >> 1) == 0 ? w.x : (k >> 1) == 1 ? w.y : (k >> 1) == 2 ? w.z : w.w;
    return (k & 1) ? (word & 0xffff0000u) : (word << 16);
}


// fp32 -> bf16 nearest-even, returned as fp32 with a zero low half; NaN
// stays NaN (quiet), infinities stay
__device__ __forceinline__ uint32_t round_to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u) return (u & 0xffff0000u) | ((u & 0xffffu) ? 0x00400000u : 0u);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xffff0000u;
}

__device__ __forceinline__ uint32_t mag16(uint32_t fbits) { return (fbits >> 16) & 0x7fffu; }

// largest bf16 magnitude (16-bit pattern) of the lane's 8 values of one row
__device__ __forceinline__ uint32_t row8_max(const u32x4& w) {
    return max_halves(pk_max_u16(pk_max_u16(abs2(w.x), abs2(w.y)), pk_max_u16(abs2(w.z), abs2(w.w))));
}

// the same value from the neighbouring lane (lane ^ 1), by DPP
__device__ __forceinline__ uint32_t pair_lane(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}

// Max over the 32 lanes of a row group of 16 per-lane 16-bit values (one
// per row), by halving exchanges (xor 16, 8, 4 keep half the rows each, xor
// 2 and 1 finish).  Returns j: the lane then holds rows 2j (low half) and
// 2j + 1 (high half) in *pair.
__device__ __forceinline__ int group_rowmax16(const uint32_t (&m)[16], uint32_t* pair) {
    const int lane = threadIdx.x & 63;
    uint32_t p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = m[2 * j] | (m[2 * j + 1] << 16);
    const bool b16 = lane & 16, b8 = lane & 8, b4 = lane & 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t send = b16 ? p[j] : p[j + 4], keep = b16 ? p[j + 4] : p[j];
        p[j] = pk_max_u16(keep, (uint32_t)__shfl_xor((int)send, 16));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t send = b8 ? p[j] : p[j + 2], keep = b8 ? p[j + 2] : p[j];
        p[j] = pk_max_u16(keep, (uint32_t)__shfl_xor((int)send, 8));
    }
    {
        const uint32_t send = b4 ? p[0] : p[1], keep = b4 ? p[1] : p[0];
        p[0] = pk_max_u16(keep, (uint32_t)__shfl_xor((int)send, 4));
    }
    p[0] = pk_max_u16(p[0], (uint32_t)__shfl_xor((int)p[0], 2));
    p[0] = pk_max_u16(p[0], (uint32_t)__shfl_xor((int)p[0], 1));
    *pair = p[0];
    return (b16 ? 4 : 0) + (b8 ? 2 : 0) + (b4 ? 1 : 0);
}

// the butterfly's largest |t| over a column block (the signs of D already
// applied to v), as the magnitude of the transformed block's largest bf16
// value: x -> RN_bf16(x / 4) is monotonic and odd, so rounding the maximum
// equals the maximum of the rounded values
__device__ __forceinline__ uint32_t rht_column_max(const u32x4 (&v)[16], int k) {
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) t[i] = __uint_as_float(col_bits(v[i], k));
#pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i & h) continue;
            const float a = t[i], b = t[i + h];
            t[i] = a + b;
            t[i + h] = a - b;
        }
    }
    float b = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) b = __builtin_fmaxf(b, __builtin_fabsf(t[i]));
    return mag16(round_to_bf16(b * 0.25f));
}

// D: row i of the lane's block negated where bit i of the mask is set (one
// xor per packed word)
__device__ __forceinline__ void apply_signs(u32x4 (&v)[16], uint32_t mask) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t sm = ((mask >> i) & 1u) ? 0x80008000u : 0u;
        v[i].x ^= sm; v[i].y ^= sm; v[i].z ^= sm; v[i].w ^= sm;
    }
}

// Pass 1: the amax of the transformed tensor, per column (col_amax [K]) or
// for the whole tensor (col_amax [1]); with ROW also the amax of x's rows
// (row_amax [M], or [1] for the tensor).  Outputs zeroed beforehand.
// Grid: (cdiv(K, 256), cdiv(M, 128 * kRhtAmaxSteps)); loads through a buffer over the
// wave's valid rows, the signs of D applied to the packed words.
template <int MODE, bool ROW>
__global__ __launch_bounds__(256) void k_rht_amax(const uint16_t* __restrict__ x, int64_t M, int64_t K, uint32_t mask,
                                                  float* __restrict__ row_amax, float* __restrict__ col_amax) {
    const int lane = threadIdx.x & 63, rg = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t c0 = (int64_t)blockIdx.x * kRhtCols + (lane & 31) * 8;
    const bool col_ok = c0 < K;
    const uint32_t xrow = (uint32_t)K * 2u;
    uint32_t xr = xrow;
    asm volatile("" : "+s"(xr));   // row offsets stay scalar
    const uint32_t vx = col_ok ? 16u * rg * xrow + (uint32_t)c0 * 2u : kOffOut;
    uint32_t m[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    uint32_t tm = 0u;   // ROW, per tensor: the rows' maximum
#pragma unroll 1
    for (int step = 0; step < kRhtAmaxSteps; ++step) {
        const int64_t wr0 = ((int64_t)blockIdx.y * kRhtAmaxSteps + step) * kRhtRows + wave * 32;
        if (wr0 >= M) break;
        // M % 16 == 0: a row group is whole or absent (its loads read zeros:
        // the buffer spans the wave's valid rows only)
        const uint32_t wrows = M - wr0 < 32 ? (uint32_t)(M - wr0) : 32u;
        const int64_t r0 = wr0 + 16 * rg;
        const __amdgpu_buffer_rsrc_t rs = rsrc(x + wr0 * K, wrows * xrow);
        u32x4 v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, vx, i * xr, 0);
        if (ROW) {
            uint32_t rm[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) rm[i] = row8_max(v[i]);
            if (MODE == ENC_TOKEN) {
                uint32_t pair;
                const int j = group_rowmax16(rm, &pair);
                if ((lane & 3) == 0 && r0 < M) {
                    if ((pair & 0xffffu) != 0u)
                        atomicMax(reinterpret_cast<uint32_t*>(row_amax + r0 + 2 * j), (pair & 0xffffu) << 16);
                    if ((pair >> 16) != 0u)
                        atomicMax(reinterpret_cast<uint32_t*>(row_amax + r0 + 2 * j + 1), pair & 0xffff0000u);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) tm = tm > rm[i] ? tm : rm[i];
            }
        }
        apply_signs(v, mask);
        // columns unrolled: a column index that varies at run time would put
        // v in scratch memory
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t b = rht_column_max(v, k);
            m[k] = m[k] > b ? m[k] : b;
        }
    }
    __shared__ uint32_t red[8][32][9];   // row group (wave, rg), lane, column (padded)
#pragma unroll
    for (int j = 0; j < 8; ++j) red[wave * 2 + rg][lane & 31][j] = m[j];
    __syncthreads();
    const int t = threadIdx.x;   // column t of the workgroup's 256
    uint32_t b = 0u;
#pragma unroll
    for (int g = 0; g < 8; ++g) b = b > red[g][t >> 3][t & 7] ? b : red[g][t >> 3][t & 7];
    if (MODE == ENC_TOKEN) {
        if ((int64_t)blockIdx.x * kRhtCols + t < K && b != 0u)
            atomicMax(reinterpret_cast<uint32_t*>(col_amax + (int64_t)blockIdx.x * kRhtCols + t), b << 16);
    } else {
        // the workgroup's maxima (columns of y; rows of x), then one atomic each
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const uint32_t ob = (uint32_t)__shfl_xor((int)b, off);
            b = b > ob ? b : ob;
            if (ROW) {
                const uint32_t ot = (uint32_t)__shfl_xor((int)tm, off);
                tm = tm > ot ? tm : ot;
            }
        }
        __shared__ uint32_t wred[4][2];
        if (lane == 0) {
            wred[wave][0] = b;
            wred[wave][1] = tm;
        }
        __syncthreads();
        if (t == 0) {
            uint32_t bc = wred[0][0], br = wred[0][1];
            for (int w = 1; w < 4; ++w) {
                bc = bc > wred[w][0] ? bc : wred[w][0];
                br = br > wred[w][1] ? br : wred[w][1];
            }
            if (bc != 0u) atomicMax(reinterpret_cast<uint32_t*>(col_amax), bc << 16);
            if (ROW && br != 0u) atomicMax(reinterpret_cast<uint32_t*>(row_amax), br << 16);
        }
    }
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

// E2M1 codes of 8 values in one word (value i in nibble i)
__device__ __forceinline__ uint32_t codes8_fast(const float (&a)[8], float yh, float yl) {
    uint32_t r = put_fp4x2<0>(0u, quot2(a[0], yh, yl), quot2(a[1], yh, yl));
    r = put_fp4x2<1>(r, quot2(a[2], yh, yl), quot2(a[3], yh, yl));
    r = put_fp4x2<2>(r, quot2(a[4], yh, yl), quot2(a[5], yh, yl));
    return put_fp4x2<3>(r, quot2(a[6], yh, yl), quot2(a[7], yh, yl));
}

__device__ __forceinline__ uint32_t codes8_exact(const float (&a)[8], const BlockScale& bs) {
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = bs.zero ? a[i] * 0.0f : a[i] / bs.r;
    uint32_t r = put_fp4x2<0>(0u, q[0], q[1]);
    r = put_fp4x2<1>(r, q[2], q[3]);
    r = put_fp4x2<2>(r, q[4], q[5]);
    return put_fp4x2<3>(r, q[6], q[7]);
}

__device__ __forceinline__ void unpack8(const u32x4& w, float (&a)[8]) {
    a[0] = bf_lo(w.x); a[1] = bf_hi(w.x); a[2] = bf_lo(w.y); a[3] = bf_hi(w.y);
    a[4] = bf_lo(w.z); a[5] = bf_hi(w.z); a[6] = bf_lo(w.w); a[7] = bf_hi(w.w);
}

// Pass 2: transform and encode.  col_q [K][M/2], col_sf [K][M/16]; with ROW
// also the rowwise cast of x itself into row_q [M][K/2], row_sf [M][K/16].
// Grid: (cdiv(K, 256), cdiv(M, 128)).
//
// Per-token outer scales are computed once per workgroup into LDS (a thread
// per row and per column of the tile).  A rowwise block is a lane pair: the
// even lane computes the block parameters of the pair's even row, the odd
// lane those of the odd row, and DPP hands them across, as in the ordinary
// cast.  The signs of D are applied to the packed words (one xor per word
// and row) after the rowwise encoding.  A column block's largest |y| is
// RN_bf16(max |t| / 4), as in the amax pass.
template <int MODE, bool ROW>
__global__ __launch_bounds__(256) void k_rht_encode(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                    uint32_t mask, const float* __restrict__ row_amax,
                                                    const float* __restrict__ col_amax, uint8_t* __restrict__ row_q,
                                                    uint8_t* __restrict__ row_sf, uint8_t* __restrict__ col_q,
                                                    uint8_t* __restrict__ col_sf) {
    const int lane = threadIdx.x & 63, rg = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool odd = lane & 1;
    const int64_t tc0 = (int64_t)blockIdx.x * kRhtCols, tr0 = (int64_t)blockIdx.y * kRhtRows;
    const int64_t c0 = tc0 + (lane & 31) * 8;
    const int rl0 = wave * 32 + 16 * rg;   // the lane's first row within the tile
    const int64_t r0 = tr0 + rl0;
    // M % 16 == 0: a row group is whole or absent; inactive lanes still take
    // part in the wave-wide path choices and the lane-pair exchange
    const bool active = c0 < K && r0 < M;
    // the wave's rows: a buffer over its valid rows (0, 16 or 32), so that an
    // absent row group reads zeros and its stores are dropped
    const int64_t wr0 = tr0 + wave * 32;
    const uint32_t wrows = wr0 >= M ? 0u : (M - wr0 < 32 ? (uint32_t)(M - wr0) : 32u);
    const uint32_t xrow = (uint32_t)K * 2u;
    uint32_t xr = xrow;
    asm volatile("" : "+s"(xr));   // row offsets stay scalar
    u32x4 v[16];
    {
        const __amdgpu_buffer_rsrc_t rs = rsrc(x + wr0 * K, wrows * xrow);
        const uint32_t vx = c0 < K ? 16u * rg * xrow + (uint32_t)c0 * 2u : kOffOut;
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, vx, i * xr, kCacheNT);
    }
    __shared__ float2 csc[MODE == ENC_TOKEN ? kRhtCols : 1];
    __shared__ float2 rsc[(MODE == ENC_TOKEN && ROW) ? kRhtRows : 1];
    if (MODE == ENC_TOKEN) {
        const int t = threadIdx.x;
        csc[t] = outer_entry(tc0 + t < K ? col_amax[tc0 + t] : 0.0f);
        if (ROW && t < kRhtRows) rsc[t] = outer_entry(tr0 + t < M ? row_amax[tr0 + t] : 0.0f);
        __syncthreads();
    }
    if (ROW) {
        const Outer rot = make_outer(MODE == ENC_TENSOR ? row_amax[0] : 0.0f);
        const uint32_t own_sel = odd ? 0x03020c0cu : 0x01000c0cu;   // own row's half to the top
        const uint32_t qrow = (uint32_t)(K / 2), srow = (uint32_t)(K / 16);
        uint32_t qr = qrow, sr = srow;
        asm volatile("" : "+s"(qr), "+s"(sr));
        const __amdgpu_buffer_rsrc_t q_rs = rsrc(row_q + wr0 * (K / 2), wrows * qrow);
        const __amdgpu_buffer_rsrc_t s_rs = rsrc(row_sf + wr0 * (K / 16), wrows * srow);
        const uint32_t vq = c0 < K ? 16u * rg * qrow + (uint32_t)c0 / 2u : kOffOut;
        const uint32_t vs = c0 < K ? (16u * rg + (odd ? 1u : 0u)) * srow + (uint32_t)c0 / 16u : kOffOut;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const u32x4 w0 = v[2 * s], w1 = v[2 * s + 1];
            const uint32_t rw0 = pk_max_u16(pk_max_u16(abs2(w0.x), abs2(w0.y)), pk_max_u16(abs2(w0.z), abs2(w0.w)));
            const uint32_t rw1 = pk_max_u16(pk_max_u16(abs2(w1.x), abs2(w1.y)), pk_max_u16(abs2(w1.z), abs2(w1.w)));
            // (row 2s | row 2s+1 << 16) over the lane's 8 columns, then the pair's 16
            uint32_t m = pk_max_u16(__builtin_amdgcn_perm(rw1, rw0, 0x05040100u),
                                    __builtin_amdgcn_perm(rw1, rw0, 0x07060302u));
            m = pk_max_u16(m, pair_lane(m));
            const Outer ro = MODE == ENC_TOKEN ? outer_from(rsc[rl0 + 2 * s + (odd ? 1 : 0)]) : rot;
            const FastBlock fb = fast_block<false>(__builtin_amdgcn_perm(m, m, own_sel), ro);
            float a0[8], a1[8];
            unpack8(w0, a0);
            unpack8(w1, a1);
            uint32_t o0, o1, code;
            if (__builtin_amdgcn_ballot_w64(ro.slow || fb.slow) == 0ull) {
                o0 = codes8_fast(a0, from_even(fb.yh), from_even(fb.yl));
                o1 = codes8_fast(a1, from_odd(fb.yh), from_odd(fb.yl));
                code = fb.code;
            } else {
                // exact path for both rows of the pair
                const float A0 = MODE == ENC_TENSOR ? row_amax[0] : (r0 < M ? row_amax[r0 + 2 * s] : 0.0f);
                const float A1 = MODE == ENC_TENSOR ? row_amax[0] : (r0 < M ? row_amax[r0 + 2 * s + 1] : 0.0f);
                const BlockScale b0 = block_scale(m & 0xffffu, outer_scale(A0));
                const BlockScale b1 = block_scale(m >> 16, outer_scale(A1));
                o0 = codes8_exact(a0, b0);
                o1 = codes8_exact(a1, b1);
                code = odd ? b1.code : b0.code;
            }
            __builtin_amdgcn_raw_buffer_store_b32(o0, q_rs, vq, (2 * s) * qr, kCacheNT);
            __builtin_amdgcn_raw_buffer_store_b32(o1, q_rs, vq, (2 * s + 1) * qr, kCacheNT);
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)code, s_rs, vs, (2 * s) * sr, 0);
        }
    }
    apply_signs(v, mask);
    // Columnwise codes are staged in LDS so that each column's 64 bytes (the
    // tile's 128 rows) leave as whole 64-byte runs: slot k * 32 + l holds
    // column 8 l + k of the tile, its 16-row group g = 2 wave + rg at byte
    // 8 g (pitch 72 bytes: two-way bank conflicts at most on the writes).
    __shared__ __attribute__((aligned(16))) uint8_t stage[kRhtCols * kRhtStagePitch];
    __shared__ __attribute__((aligned(8))) uint8_t sstage[kRhtCols * 8];   // scale codes, slot-major
    const Outer cot = make_outer(MODE == ENC_TENSOR ? col_amax[0] : 0.0f);
#pragma unroll
    for (int k = 0; k < 8; ++k) {   // unrolled (see k_rht_amax)
        float t[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) t[i] = __uint_as_float(col_bits(v[i], k));
#pragma unroll
        for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (i & h) continue;
                const float a = t[i], b = t[i + h];
                t[i] = a + b;
                t[i + h] = a - b;
            }
        }
        float bmx = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) bmx = __builtin_fmaxf(bmx, __builtin_fabsf(t[i]));
        // y = RN_bf16(t / 4), and the block's largest |y| the same way
        float y[16];
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            const uint32_t w = bf16x2_rne(t[i] * 0.25f, t[i + 1] * 0.25f);
            y[i] = bf_lo(w);
            y[i + 1] = bf_hi(w);
        }
        const uint32_t bb = bf16x2_rne(bmx * 0.25f, 0.0f) << 16;
        const Outer co = MODE == ENC_TOKEN ? outer_from(csc[(lane & 31) * 8 + k]) : cot;
        const FastBlock fb = fast_block<false>(bb, co);
        const float (&ylo)[8] = *reinterpret_cast<const float (*)[8]>(&y[0]);
        const float (&yhi)[8] = *reinterpret_cast<const float (*)[8]>(&y[8]);
        uint32_t lo, hi, code;
        if (__builtin_amdgcn_ballot_w64(co.slow || fb.slow) == 0ull) {
            lo = codes8_fast(ylo, fb.yh, fb.yl);
            hi = codes8_fast(yhi, fb.yh, fb.yl);
            code = fb.code & 0xffu;
        } else {
            // exact path: IEEE block scale and element divisions
            const float A = MODE == ENC_TENSOR ? col_amax[0] : (active ? col_amax[c0 + k] : 0.0f);
            const BlockScale bs = block_scale(bb >> 16, outer_scale(A));
            lo = codes8_exact(ylo, bs);
            hi = codes8_exact(yhi, bs);
            code = bs.code;
        }
        *reinterpret_cast<u32x2*>(stage + (k * 32 + (lane & 31)) * kRhtStagePitch + 8 * (2 * wave + rg)) =
            u32x2{lo, hi};
        sstage[(k * 32 + (lane & 31)) * 8 + 2 * wave + rg] = (uint8_t)code;
    }
    __syncthreads();
    // thread t writes the 8 scale codes of slot t (one 8-byte store where the
    // tile's rows are whole and the address allows it)
    {
        const int t = threadIdx.x;
        const int64_t col = tc0 + 8 * (t & 31) + (t >> 5);
        if (col < K) {
            uint8_t* dst = col_sf + col * (M / 16) + tr0 / 16;
            const uint8_t* src = sstage + t * 8;
            if (tr0 + kRhtRows <= M && (reinterpret_cast<uintptr_t>(dst) & 7u) == 0)
                *reinterpret_cast<u32x2*>(dst) = *reinterpret_cast<const u32x2*>(src);
            else
                for (int q = 0; q < 8; ++q)
                    if (tr0 + 16 * q < M) dst[q] = src[q];
        }
    }
    // thread t writes 8-byte piece g = t % 8 (rows 16 g .. 16 g + 15 of the
    // tile) of slots t / 8 + 32 j: eight lanes cover one column's run
    const int g = threadIdx.x & 7, l = threadIdx.x >> 3;
    const int64_t tr = tr0 + 16 * g;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t col = tc0 + 8 * l + j;
        if (col < K && tr < M)
            *reinterpret_cast<u32x2*>(col_q + col * (M / 2) + tr / 2) =
                *reinterpret_cast<const u32x2*>(stage + (j * 32 + l) * kRhtStagePitch + 8 * g);
    }
}

}  // namespace

hipError_t launch_rht(int mode, const uint16_t* x, int64_t M, int64_t K, uint32_t mask, float* row_amax,
                      float* col_amax, uint8_t* row_q, uint8_t* row_sf, uint8_t* col_q, uint8_t* col_sf, hipStream_t st,
                      hipEvent_t ev0, hipEvent_t ev1) {
    if (M <= 0 || K <= 0) return hipSuccess;
    const unsigned gx = (unsigned)((K + kRhtCols - 1) / kRhtCols);
    const dim3 ga(gx, (unsigned)((M + kRhtRows * kRhtAmaxSteps - 1) / (kRhtRows * kRhtAmaxSteps)));
    const dim3 ge(gx, (unsigned)((M + kRhtRows - 1) / kRhtRows));
#define NVFP4_RHT_LAUNCH(MD, R)                                                                                     \
    do {                                                                                                          \
        hipLaunchKernelGGL((k_rht_amax<MD, R>), ga, dim3(256), 0, st, x, M, K, mask, row_amax, col_amax);         \
        hipExtLaunchKernelGGL((k_rht_encode<MD, R>), ge, dim3(256), 0, st, ev0, ev1, 0, x, M, K, mask,            \
                              (const float*)row_amax, (const float*)col_amax, row_q, row_sf, col_q, col_sf);      \
    } while (0)
    const bool row = row_q != nullptr;
    if (mode == ENC_TOKEN) {
        if (row) NVFP4_RHT_LAUNCH(ENC_TOKEN, true);
        else NVFP4_RHT_LAUNCH(ENC_TOKEN, false);
    } else {
        if (row) NVFP4_RHT_LAUNCH(ENC_TENSOR, true);
        else NVFP4_RHT_LAUNCH(ENC_TENSOR, false);
    }
#undef NVFP4_RHT_LAUNCH
    return hipGetLastError();
}

}  // namespace nvfp4
