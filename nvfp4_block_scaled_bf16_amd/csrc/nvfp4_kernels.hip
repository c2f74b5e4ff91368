// nvfp4_kernels.hip -- general-path HIP kernels of the bf16 -> NVFP4 cast for
// gfx950: outer amax, encode (rowwise and columnwise from one read), 16x16
// tiles, grouped experts, dequantize and the decayed accumulator.  They serve
// every shape the C ABI accepts; large aligned per-token and per-tensor casts
// take the fused path in nvfp4_fused.hip instead.
//
// Work decomposition shared by the amax and encode kernels: a lane owns a
// 16-row x 8-column sub-block (sixteen 16-byte loads, one per row), so a
// wave covers 16 rows x 512 columns and reads 1 KB of one row per load
// instruction.  A lane's 8 columns x 16 rows are eight complete columnwise
// blocks; the 16 rows hold half of a rowwise block each, the other half
// sitting in the neighbouring lane (lanes 2j and 2j+1 exchange maxima).
#include "nvfp4_device.hpp"
#include "nvfp4_internal.h"

namespace nvfp4 {

constexpr int kTileCols = 512;     // columns per workgroup tile (64 lanes x 8)
constexpr int kAmaxRows = 256;     // rows per workgroup tile in the amax pass
constexpr int kEncRows = 256;      // rows per workgroup tile in the encode pass

// --------------------------------------------------------------- utilities

__global__ void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t s = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += s) p[i] = v;
}

// max of non-negative floats through their bit patterns
__device__ __forceinline__ void atomic_max_mag(float* p, uint32_t mag16) {
    if (mag16 != 0u) atomicMax(reinterpret_cast<uint32_t*>(p), mag16 << 16);
}

// load 16 rows x 8 bf16 (one 16-byte word per row) of a lane's sub-block;
// rows at or beyond row_end, or a lane past the last column, read zeros
__device__ __forceinline__ void load_subblock(const uint16_t* __restrict__ x, int64_t K, int64_t r0,
                                              int64_t row_end, int64_t c0, bool col_ok, u32x4 v[16]) {
    const u32x4* base = reinterpret_cast<const u32x4*>(x + r0 * K + c0);
    const int64_t stride = K / 8;  // in 16-byte words
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (col_ok && r0 + i < row_end) v[i] = __builtin_nontemporal_load(base + i * stride);
        else v[i] = u32x4{0u, 0u, 0u, 0u};
    }
}

// Max over the wave of 16 per-lane 16-bit values (one per row), by halving
// exchanges: after the xor-32/16/8 steps each lane holds a pair of rows, the
// xor-4/2/1 steps finish the reduction.  Returns the pair index j (rows 2j,
// 2j+1 in the low/high half of *pair) that this lane now holds.
__device__ __forceinline__ int wave_rowmax16(const uint32_t m[16], uint32_t* pair) {
    const int lane = threadIdx.x & 63;
    uint32_t p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = m[2 * j] | (m[2 * j + 1] << 16);
    const bool b32 = lane & 32, b16 = lane & 16, b8 = lane & 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t send = b32 ? p[j] : p[j + 4];
        uint32_t keep = b32 ? p[j + 4] : p[j];
        p[j] = pk_max_u16(keep, (uint32_t)__shfl_xor((int)send, 32));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        uint32_t send = b16 ? p[j] : p[j + 2];
        uint32_t keep = b16 ? p[j + 2] : p[j];
        p[j] = pk_max_u16(keep, (uint32_t)__shfl_xor((int)send, 16));
    }
    {
        uint32_t send = b8 ? p[0] : p[1];
        uint32_t keep = b8 ? p[1] : p[0];
        p[0] = pk_max_u16(keep, (uint32_t)__shfl_xor((int)send, 8));
    }
    p[0] = pk_max_u16(p[0], (uint32_t)__shfl_xor((int)p[0], 4));
    p[0] = pk_max_u16(p[0], (uint32_t)__shfl_xor((int)p[0], 2));
    p[0] = pk_max_u16(p[0], (uint32_t)__shfl_xor((int)p[0], 1));
    *pair = p[0];
    return (b32 ? 4 : 0) + (b16 ? 2 : 0) + (b8 ? 1 : 0);
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, d);
        v = v > o ? v : o;
    }
    return v;
}

// ---------------------------------------------------------------- amax pass

// KIND: AMAX_TENSOR (one max over everything into t0 and/or t1),
// AMAX_TOKEN (row maxima into row_amax, column maxima into col_amax, either
// may be null), AMAX_GROUPED (row maxima as AMAX_TOKEN, column maxima per
// expert into col_amax[e][K]).
// Outputs must hold zeros (or smaller values) on entry: they are combined
// with atomic max.  Rows [row_begin, row_end) are covered.
template <int KIND>
__global__ __launch_bounds__(256) void k_amax(const uint16_t* __restrict__ x, int64_t K,
                                              int64_t row_begin, int64_t row_end,
                                              float* __restrict__ row_amax, float* __restrict__ col_amax,
                                              float* __restrict__ t0, float* __restrict__ t1, GroupTable gt) {
    __shared__ uint32_t red[4][64][4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t c0 = (int64_t)blockIdx.x * kTileCols + lane * 8;
    const bool col_ok = c0 < K;
    const int64_t rb = row_begin + (int64_t)blockIdx.y * kAmaxRows + wave * (kAmaxRows / 4);
    uint32_t cm[4] = {0u, 0u, 0u, 0u};
    uint32_t tm = 0u;
    int cur_group = -1;
    for (int s = 0; s < kAmaxRows / 4; s += 16) {
        const int64_t r0 = rb + s;
        if (r0 >= row_end) break;
        if (KIND == AMAX_GROUPED) {
            int g = group_of_row(gt, r0);
            if (g != cur_group) {
                if (cur_group >= 0 && col_ok) {
                    float* dst = col_amax + (int64_t)(gt.first + cur_group) * K + c0;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        atomic_max_mag(dst + 2 * k, cm[k] & 0xffffu);
                        atomic_max_mag(dst + 2 * k + 1, cm[k] >> 16);
                        cm[k] = 0u;
                    }
                }
                cur_group = g;
            }
        }
        u32x4 v[16];
        load_subblock(x, K, r0, row_end, c0, col_ok, v);
        uint32_t rm[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            uint32_t a = pk_max_u16(pk_max_u16(abs2(v[i].x), abs2(v[i].y)), pk_max_u16(abs2(v[i].z), abs2(v[i].w)));
            rm[i] = max_halves(a);
            cm[0] = pk_max_u16(cm[0], abs2(v[i].x));
            cm[1] = pk_max_u16(cm[1], abs2(v[i].y));
            cm[2] = pk_max_u16(cm[2], abs2(v[i].z));
            cm[3] = pk_max_u16(cm[3], abs2(v[i].w));
        }
        if ((KIND == AMAX_TOKEN || KIND == AMAX_GROUPED) && row_amax != nullptr) {
            uint32_t pair;
            int j = wave_rowmax16(rm, &pair);
            if ((lane & 7) == 0) {
                if (r0 + 2 * j < row_end) atomic_max_mag(row_amax + r0 + 2 * j, pair & 0xffffu);
                if (r0 + 2 * j + 1 < row_end) atomic_max_mag(row_amax + r0 + 2 * j + 1, pair >> 16);
            }
        }
        if (KIND == AMAX_TENSOR) {
#pragma unroll
            for (int i = 0; i < 16; ++i) tm = tm > rm[i] ? tm : rm[i];
        }
    }
    if (KIND == AMAX_TENSOR) {
        tm = wave_max(tm);
        __shared__ uint32_t tred[4];
        if (lane == 0) tred[wave] = tm;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t m = tred[0];
            for (int w = 1; w < 4; ++w) m = m > tred[w] ? m : tred[w];
            if (t0) atomic_max_mag(t0, m);
            if (t1) atomic_max_mag(t1, m);
        }
        return;
    }
    if (KIND == AMAX_GROUPED) {
        if (cur_group >= 0 && col_ok) {
            float* dst = col_amax + (int64_t)(gt.first + cur_group) * K + c0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                atomic_max_mag(dst + 2 * k, cm[k] & 0xffffu);
                atomic_max_mag(dst + 2 * k + 1, cm[k] >> 16);
            }
        }
        return;
    }
    if (col_amax != nullptr) {
        // combine the four waves' column maxima, then one atomic per column
#pragma unroll
        for (int k = 0; k < 4; ++k) red[wave][lane][k] = cm[k];
        __syncthreads();
        if (wave == 0 && col_ok) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                uint32_t m = pk_max_u16(pk_max_u16(red[0][lane][k], red[1][lane][k]),
                                        pk_max_u16(red[2][lane][k], red[3][lane][k]));
                atomic_max_mag(col_amax + c0 + 2 * k, m & 0xffffu);
                atomic_max_mag(col_amax + c0 + 2 * k + 1, m >> 16);
            }
        }
    }
}

// -------------------------------------------------------------- encode pass

// exact per-element quotient for the slow path
__device__ __forceinline__ float quotient_exact(float a, const BlockScale& bs) {
    return bs.zero ? a * 0.0f : a / bs.r;
}

// element k (0..7) of a 16x8 sub-block row held as 4 words
__device__ __forceinline__ float elem(const u32x4& w, int k) {
    const uint32_t word = (k >> 1) == 0 ? w.x : (k >> 1) == 1 ? w.y : (k >> 1) == 2 ? w.z : w.w;
    return (k & 1) ? bf_hi(word) : bf_lo(word);
}

// DPP: value of the neighbouring lane (lane ^ 1)
__device__ __forceinline__ uint32_t from_pair(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t rowmax_word(const u32x4& w) {
    return pk_max_u16(pk_max_u16(abs2(w.x), abs2(w.y)), pk_max_u16(abs2(w.z), abs2(w.w)));
}

// Where a lane's sub-block results go.  Columnwise data of column c, rows
// [r0, r0+16) of a vector of length m_len starting at row grow0.
struct SubDst {
    uint8_t* row_q; uint8_t* row_sf; uint8_t* col_q; uint8_t* col_sf;
    int64_t K, r0, c0, row_end, m_len, grow0;
    bool col_ok, even;
};

__device__ __forceinline__ void store_row(const SubDst& d, int i, uint32_t q, uint32_t code) {
    const int64_t r = d.r0 + i;
    if (d.col_ok && r < d.row_end) {
        *reinterpret_cast<uint32_t*>(d.row_q + r * (d.K / 2) + d.c0 / 2) = q;
        if (d.even) d.row_sf[r * (d.K / 16) + d.c0 / 16] = (uint8_t)code;
    }
}

__device__ __forceinline__ void store_row_pair(const SubDst& d, int i, uint32_t q0, uint32_t q1, uint32_t own_code) {
    if (!d.col_ok) return;
    const int64_t r = d.r0 + i;
    if (r < d.row_end) *reinterpret_cast<uint32_t*>(d.row_q + r * (d.K / 2) + d.c0 / 2) = q0;
    if (r + 1 < d.row_end) *reinterpret_cast<uint32_t*>(d.row_q + (r + 1) * (d.K / 2) + d.c0 / 2) = q1;
    const int64_t ro = d.even ? r : r + 1;
    if (ro < d.row_end) d.row_sf[ro * (d.K / 16) + d.c0 / 16] = (uint8_t)own_code;
}

__device__ __forceinline__ void store_col(const SubDst& d, int j, uint32_t lo, uint32_t hi, uint32_t code) {
    if (!d.col_ok) return;
    const int64_t c = d.c0 + j;
    uint8_t* qb = d.col_q + d.grow0 * d.K / 2;
    uint8_t* sb = d.col_sf + d.grow0 * d.K / 16;
    *reinterpret_cast<u32x2*>(qb + c * (d.m_len / 2) + (d.r0 - d.grow0) / 2) = u32x2{lo, hi};
    sb[c * (d.m_len / 16) + (d.r0 - d.grow0) / 16] = (uint8_t)code;
}

// Fast encode and store of one lane's 16x8 sub-block.  Row outer scales are
// wave-uniform (rowS/rowYS per row, a bit mask of rows needing the exact
// path); colO are this lane's 8 columns; tileO the tensor's (16x16 tiles).
// The two lanes of a pair share every rowwise block: each computes the
// parameters of one row of every row pair (row 2s + parity) and the pair
// swaps them.  Returns true if some block needs the exact path, in which
// case the caller re-encodes the sub-block exactly over what was stored.
template <bool ROW, bool COL, bool TILE, bool SAT>
__device__ __forceinline__ bool encode_fast(const u32x4 v[16], const float* rowS, const float* rowYS,
                                            uint32_t row_slow, const Outer* colO, const Outer& tileO,
                                            const SubDst& d) {
    const bool odd = !d.even;
    bool slow = false;
    FastBlock cb[8];
    FastBlock tb;
    if (TILE) {
        uint32_t m = 0u;
#pragma unroll
        for (int i = 0; i < 16; ++i) m = pk_max_u16(m, rowmax_word(v[i]));
        m = pk_max_u16(m, from_pair(m));
        tb = fast_block<SAT>(max_halves(m), tileO);
        slow = tb.slow;
    } else if (COL) {
        uint32_t cm[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            cm[0] = pk_max_u16(cm[0], abs2(v[i].x));
            cm[1] = pk_max_u16(cm[1], abs2(v[i].y));
            cm[2] = pk_max_u16(cm[2], abs2(v[i].z));
            cm[3] = pk_max_u16(cm[3], abs2(v[i].w));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            cb[j] = fast_block<SAT>((j & 1) ? (cm[j >> 1] >> 16) : (cm[j >> 1] & 0xffffu), colO[j]);
            slow |= cb[j].slow;
        }
    }
    uint32_t cq[8][2];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
        float a[2][8];
#pragma unroll
        for (int k = 0; k < 8; ++k) { a[0][k] = elem(v[i], k); a[1][k] = elem(v[i + 1], k); }
        if (ROW) {
            float rr[2], ry[2];
            uint32_t own_code;
            if (TILE) {
                rr[0] = rr[1] = tb.r; ry[0] = ry[1] = tb.y; own_code = tb.code;
            } else {
                uint32_t f0 = rowmax_word(v[i]), f1 = rowmax_word(v[i + 1]);
                f0 = pk_max_u16(f0, from_pair(f0));
                f1 = pk_max_u16(f1, from_pair(f1));
                Outer ro;
                ro.S = odd ? rowS[i + 1] : rowS[i];
                ro.yS = odd ? rowYS[i + 1] : rowYS[i];
                ro.slow = (row_slow >> (i + (odd ? 1 : 0))) & 1u;
                const FastBlock f = fast_block<SAT>(max_halves(odd ? f1 : f0), ro);
                slow |= f.slow;
                const float pr = __uint_as_float(from_pair(__float_as_uint(f.r)));
                const float py = __uint_as_float(from_pair(__float_as_uint(f.y)));
                rr[0] = odd ? pr : f.r; ry[0] = odd ? py : f.y;
                rr[1] = odd ? f.r : pr; ry[1] = odd ? f.y : py;
                own_code = f.code;
            }
            uint32_t w[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t q = 0u;
                q = put_fp4x2<0>(q, div_fast(a[h][0], rr[h], ry[h]), div_fast(a[h][1], rr[h], ry[h]));
                q = put_fp4x2<1>(q, div_fast(a[h][2], rr[h], ry[h]), div_fast(a[h][3], rr[h], ry[h]));
                q = put_fp4x2<2>(q, div_fast(a[h][4], rr[h], ry[h]), div_fast(a[h][5], rr[h], ry[h]));
                q = put_fp4x2<3>(q, div_fast(a[h][6], rr[h], ry[h]), div_fast(a[h][7], rr[h], ry[h]));
                w[h] = q;
            }
            store_row_pair(d, i, w[0], w[1], own_code);
        }
        if (COL) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const FastBlock& f = TILE ? tb : cb[j];
                const float q0 = div_fast(a[0][j], f.r, f.y), q1 = div_fast(a[1][j], f.r, f.y);
                uint32_t& w = cq[j][i >> 3];
                const int byte = (i >> 1) & 3;
                if (byte == 0) w = put_fp4x2<0>(0u, q0, q1);
                else if (byte == 1) w = put_fp4x2<1>(w, q0, q1);
                else if (byte == 2) w = put_fp4x2<2>(w, q0, q1);
                else w = put_fp4x2<3>(w, q0, q1);
            }
        }
    }
    if (COL) {
#pragma unroll
        for (int j = 0; j < 8; ++j) store_col(d, j, cq[j][0], cq[j][1], TILE ? tb.code : cb[j].code);
    }
    return slow;
}

// Exact encode and store of a sub-block with IEEE divisions throughout,
// re-reading the data.  rowA: amax of row r0+i for lanes 0..15 (lane i holds
// row i's), broadcast here; colA: this lane's 8 column amax; tileA: tensor's.
template <bool ROW, bool COL, bool TILE>
__device__ __noinline__ void encode_exact(const uint16_t* __restrict__ x, float rowA_lane, float colA0, float colA1,
                                          float colA2, float colA3, float colA4, float colA5, float colA6,
                                          float colA7, float tileA, SubDst d) {
    u32x4 v[16];
    load_subblock(x, d.K, d.r0, d.row_end, d.c0, d.col_ok, v);
    const float colA[8] = {colA0, colA1, colA2, colA3, colA4, colA5, colA6, colA7};
    if (TILE) {
        uint32_t m = 0u;
        for (int i = 0; i < 16; ++i) m = pk_max_u16(m, rowmax_word(v[i]));
        m = pk_max_u16(m, from_pair(m));
        const BlockScale bs = block_scale(max_halves(m), outer_scale(tileA));
        for (int i = 0; i < 16; ++i) {
            uint32_t w = 0u;
            for (int k = 0; k < 8; k += 2)
                w |= (__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, quotient_exact(elem(v[i], k), bs),
                                                              quotient_exact(elem(v[i], k + 1), bs), 1.0f, 0) & 0xffu) << (4 * k);
            if (ROW) store_row(d, i, w, bs.code);
        }
        if (COL)
            for (int j = 0; j < 8; ++j) {
                uint32_t lohi[2] = {0u, 0u};
                for (int i = 0; i < 16; i += 2)
                    lohi[i >> 3] |= (__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, quotient_exact(elem(v[i], j), bs),
                                                                         quotient_exact(elem(v[i + 1], j), bs), 1.0f, 0) & 0xffu) << (8 * ((i >> 1) & 3));
                store_col(d, j, lohi[0], lohi[1], bs.code);
            }
        return;
    }
    if (ROW) {
        for (int i = 0; i < 16; ++i) {
            const float A = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rowA_lane), i));
            uint32_t hw = rowmax_word(v[i]);
            hw = pk_max_u16(hw, from_pair(hw));
            const BlockScale bs = block_scale(max_halves(hw), outer_scale(A));
            uint32_t w = 0u;
            for (int k = 0; k < 8; k += 2)
                w |= (__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, quotient_exact(elem(v[i], k), bs),
                                                              quotient_exact(elem(v[i], k + 1), bs), 1.0f, 0) & 0xffu) << (4 * k);
            store_row(d, i, w, bs.code);
        }
    }
    if (COL) {
        for (int j = 0; j < 8; ++j) {
            uint32_t m = 0u;
            for (int i = 0; i < 16; ++i) {
                const uint32_t e = (__float_as_uint(elem(v[i], j)) >> 16) & 0x7fffu;
                m = e > m ? e : m;
            }
            const BlockScale bs = block_scale(m, outer_scale(colA[j]));
            uint32_t lohi[2] = {0u, 0u};
            for (int i = 0; i < 16; i += 2)
                lohi[i >> 3] |= (__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, quotient_exact(elem(v[i], j), bs),
                                                                     quotient_exact(elem(v[i + 1], j), bs), 1.0f, 0) & 0xffu) << (8 * ((i >> 1) & 3));
            store_col(d, j, lohi[0], lohi[1], bs.code);
        }
    }
}

// MODE: ENC_TENSOR (row_amax[0] / col_amax[0] for every vector), ENC_TOKEN
// (row_amax[r], col_amax[c]), ENC_TILE (16x16 tiles, tensor amax in
// row_amax[0] or col_amax[0]; also fills row_amax[1..M) and col_amax[1..K)
// with it), ENC_GROUPED (rowwise per-token; columnwise per expert with
// col_amax[e][K] and per-expert output slabs).  A workgroup covers 256 rows
// x 512 columns; each wave walks four 16-row sub-blocks.
template <int MODE, bool ROW, bool COL, bool SAT>
__global__ __launch_bounds__(256) void k_encode(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                int64_t row_begin, int64_t row_end,
                                                const float* __restrict__ row_amax, const float* __restrict__ col_amax,
                                                uint8_t* __restrict__ row_q, uint8_t* __restrict__ row_sf,
                                                uint8_t* __restrict__ col_q, uint8_t* __restrict__ col_sf,
                                                float* __restrict__ fill_row, float* __restrict__ fill_col,
                                                GroupTable gt) {
    constexpr bool TILE = MODE == ENC_TILE;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    SubDst d;
    d.row_q = row_q; d.row_sf = row_sf; d.col_q = col_q; d.col_sf = col_sf;
    d.K = K; d.c0 = (int64_t)blockIdx.x * kTileCols + lane * 8; d.row_end = row_end;
    d.m_len = M; d.grow0 = 0; d.col_ok = d.c0 < K; d.even = (lane & 1) == 0;
    const int64_t rbase = row_begin + (int64_t)blockIdx.y * kEncRows + wave * (kEncRows / 4);
    float tileA = 0.0f;
    if (TILE) {
        tileA = row_amax ? row_amax[0] : col_amax[0];
        const int64_t gid = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
        const int64_t gsz = (int64_t)gridDim.x * gridDim.y * blockDim.x;
        if (fill_row) for (int64_t i = 1 + gid; i < M; i += gsz) fill_row[i] = tileA;
        if (fill_col) for (int64_t i = 1 + gid; i < K; i += gsz) fill_col[i] = tileA;
    }
    const Outer tileO = make_outer(tileA);

    // columnwise outer scales of this lane's 8 columns
    float colA[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    Outer colO[8];
    int cur_group = -1;
    if (COL && !TILE && MODE != ENC_GROUPED) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            colA[j] = (MODE == ENC_TENSOR) ? col_amax[0] : (d.col_ok ? col_amax[d.c0 + j] : 0.0f);
            colO[j] = make_outer(colA[j]);
        }
    }
    // per-tensor rowwise outer scale
    float rowA_t = 0.0f;
    Outer rowO_t;
    if (ROW && MODE == ENC_TENSOR) { rowA_t = row_amax[0]; }
    rowO_t = make_outer(rowA_t);

    for (int sb = 0; sb < kEncRows / 64; ++sb) {
        d.r0 = rbase + 16 * sb;
        if (d.r0 >= row_end) break;
        if (COL && MODE == ENC_GROUPED) {
            const int g = group_of_row(gt, d.r0);
            if (g != cur_group) {
                cur_group = g;
                d.m_len = gt.cnt[g];
                d.grow0 = gt.off[g];
                const int64_t base = (int64_t)(gt.first + g) * K;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    colA[j] = d.col_ok ? col_amax[base + d.c0 + j] : 0.0f;
                    colO[j] = make_outer(colA[j]);
                }
            }
        }
        u32x4 v[16];
        load_subblock(x, K, d.r0, row_end, d.c0, d.col_ok, v);

        // rowwise outer scales of the 16 rows: lanes 0..15 compute one row
        // each; S and 1/S are broadcast through readlane, flags through ballot
        float rowS[16], rowYS[16];
        uint32_t row_slow = 0u;
        float rowA_lane = rowA_t;
        if (ROW && !TILE) {
            Outer mine = rowO_t;
            if (MODE != ENC_TENSOR) {
                const int64_t rr = d.r0 + (lane & 15);
                rowA_lane = rr < row_end ? row_amax[rr] : 0.0f;
                mine = make_outer(rowA_lane);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                rowS[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine.S), i));
                rowYS[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine.yS), i));
            }
            row_slow = (uint32_t)__builtin_amdgcn_ballot_w64(mine.slow) & 0xffffu;
        }

        const bool slow = encode_fast<ROW, COL, TILE, SAT>(v, rowS, rowYS, row_slow, colO, tileO, d);
        if (__builtin_amdgcn_ballot_w64(slow) != 0ull)
            encode_exact<ROW, COL, TILE>(x, rowA_lane, colA[0], colA[1], colA[2], colA[3], colA[4], colA[5],
                                         colA[6], colA[7], tileA, d);
    }
}

// ---------------------------------------------------------------- dequantize

// one thread per 16-element block: out = (+/-) g * (decode(sf) * (A / 2688))
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ q, const uint8_t* __restrict__ sf,
                                                 const float* __restrict__ amax, int64_t R, int64_t C,
                                                 int amax_per_row, float* __restrict__ out) {
    const int64_t nb = C / 16;
    int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; t < R * nb; t += stride) {
        const int64_t r = t / nb, j = t - r * nb;
        const float S = outer_scale(amax[amax_per_row ? r : 0]);
        const float ratio = e4m3_value(sf[t]) * S;
        const u32x2 w = *reinterpret_cast<const u32x2*>(q + r * (C / 2) + 8 * j);
        float o[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t byte = ((i < 8 ? w.x : w.y) >> (8 * ((i >> 1) & 3))) & 0xffu;
            const uint32_t nib = (i & 1) ? (byte >> 4) : (byte & 0xfu);
            const uint32_t c = nib & 7u;
            // E2M1 magnitude: 0, 0.5, then 2^(e-1) * (1 + m/2) for c >= 2
            const uint32_t gbits = c < 2u ? (c ? 0x3F000000u : 0u) : ((((c >> 1) + 126u) << 23) | ((c & 1u) << 22));
            const float g = __uint_as_float(gbits | ((nib & 8u) << 28));
            o[i] = g * ratio;
        }
        float4* dst = reinterpret_cast<float4*>(out + r * C + 16 * j);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
    }
}

// --------------------------------------------------------- decayed maximum

__global__ void k_accumulate(float* __restrict__ buf, const float* __restrict__ obs, int64_t n, float decay) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t s = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += s) {
        const float t = buf[i] * decay;
        const float o = obs[i];
        buf[i] = o > t ? o : t;
    }
}

// one workgroup: m = max(obs), then buf[0] = max(buf[0] * decay, m)
__global__ __launch_bounds__(256) void k_accumulate_reduce(float* __restrict__ buf, const float* __restrict__ obs,
                                                           int64_t n, float decay) {
    __shared__ float red[4];
    float m = 0.0f;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) m = obs[i] > m ? obs[i] : m;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const float o = __shfl_xor(m, d);
        m = o > m ? o : m;
    }
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 4; ++w) m = red[w] > m ? red[w] : m;
        const float t = buf[0] * decay;
        buf[0] = m > t ? m : t;
    }
}

// ------------------------------------------------------------------ launchers

static inline unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    unsigned grid = cdiv(n, 256);
    if (grid > 4096) grid = 4096;
    hipLaunchKernelGGL(k_fill_u32, dim3(grid), dim3(256), 0, st, reinterpret_cast<uint32_t*>(p), n, __builtin_bit_cast(uint32_t, v));
    return hipGetLastError();
}

hipError_t launch_amax(int kind, const uint16_t* x, int64_t K, int64_t row_begin, int64_t row_end,
                       float* row_amax, float* col_amax, float* t0, float* t1, const GroupTable& gt,
                       hipStream_t st) {
    if (row_end <= row_begin || K <= 0) return hipSuccess;
    dim3 grid(cdiv(K, kTileCols), cdiv(row_end - row_begin, kAmaxRows));
    switch (kind) {
    case AMAX_TENSOR:
        hipLaunchKernelGGL(k_amax<AMAX_TENSOR>, grid, dim3(256), 0, st, x, K, row_begin, row_end, row_amax, col_amax, t0, t1, gt);
        break;
    case AMAX_TOKEN:
        hipLaunchKernelGGL(k_amax<AMAX_TOKEN>, grid, dim3(256), 0, st, x, K, row_begin, row_end, row_amax, col_amax, t0, t1, gt);
        break;
    default:
        hipLaunchKernelGGL(k_amax<AMAX_GROUPED>, grid, dim3(256), 0, st, x, K, row_begin, row_end, row_amax, col_amax, t0, t1, gt);
        break;
    }
    return hipGetLastError();
}

template <int MODE, bool SAT>
static void launch_encode_mode(bool row, bool col, dim3 grid, hipStream_t st, const uint16_t* x, int64_t M, int64_t K,
                               int64_t rb, int64_t re, const float* ra, const float* ca, uint8_t* rq, uint8_t* rs,
                               uint8_t* cq, uint8_t* cs, float* fr, float* fc, const GroupTable& gt) {
    if (row && col)
        hipLaunchKernelGGL((k_encode<MODE, true, true, SAT>), grid, dim3(256), 0, st, x, M, K, rb, re, ra, ca, rq, rs, cq, cs, fr, fc, gt);
    else if (row)
        hipLaunchKernelGGL((k_encode<MODE, true, false, SAT>), grid, dim3(256), 0, st, x, M, K, rb, re, ra, ca, rq, rs, cq, cs, fr, fc, gt);
    else
        hipLaunchKernelGGL((k_encode<MODE, false, true, SAT>), grid, dim3(256), 0, st, x, M, K, rb, re, ra, ca, rq, rs, cq, cs, fr, fc, gt);
}

hipError_t launch_encode(int mode, bool row, bool col, bool caller_amax, const uint16_t* x, int64_t M, int64_t K,
                         int64_t row_begin, int64_t row_end, const float* row_amax, const float* col_amax,
                         uint8_t* row_q, uint8_t* row_sf, uint8_t* col_q, uint8_t* col_sf,
                         float* fill_row, float* fill_col, const GroupTable& gt, hipStream_t st) {
    if (row_end <= row_begin || K <= 0 || (!row && !col)) return hipSuccess;
    dim3 grid(cdiv(K, kTileCols), cdiv(row_end - row_begin, kEncRows));
#define NVFP4_ENC_ARGS row, col, grid, st, x, M, K, row_begin, row_end, row_amax, col_amax, row_q, row_sf, col_q, col_sf, fill_row, fill_col, gt
    if (caller_amax) {
        // amax from the caller: scales may saturate
        if (mode == ENC_TENSOR) launch_encode_mode<ENC_TENSOR, true>(NVFP4_ENC_ARGS);
        else launch_encode_mode<ENC_TOKEN, true>(NVFP4_ENC_ARGS);
    } else {
        switch (mode) {
        case ENC_TENSOR: launch_encode_mode<ENC_TENSOR, false>(NVFP4_ENC_ARGS); break;
        case ENC_TOKEN: launch_encode_mode<ENC_TOKEN, false>(NVFP4_ENC_ARGS); break;
        case ENC_TILE: launch_encode_mode<ENC_TILE, false>(NVFP4_ENC_ARGS); break;
        default: launch_encode_mode<ENC_GROUPED, false>(NVFP4_ENC_ARGS); break;
        }
    }
#undef NVFP4_ENC_ARGS
    return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* q, const uint8_t* sf, const float* amax, int64_t R, int64_t C,
                          int amax_per_row, float* out, hipStream_t st) {
    const int64_t blocks = R * (C / 16);
    if (blocks <= 0) return hipSuccess;
    unsigned grid = cdiv(blocks, 256);
    if (grid > 16384) grid = 16384;
    hipLaunchKernelGGL(k_dequant, dim3(grid), dim3(256), 0, st, q, sf, amax, R, C, amax_per_row, out);
    return hipGetLastError();
}

hipError_t launch_accumulate(float* buf, const float* obs, int64_t n, float decay, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    unsigned grid = cdiv(n, 256);
    if (grid > 4096) grid = 4096;
    hipLaunchKernelGGL(k_accumulate, dim3(grid), dim3(256), 0, st, buf, obs, n, decay);
    return hipGetLastError();
}

hipError_t launch_accumulate_reduce(float* buf, const float* obs, int64_t n, float decay, hipStream_t st) {
    hipLaunchKernelGGL(k_accumulate_reduce, dim3(1), dim3(256), 0, st, buf, obs, n, decay);
    return hipGetLastError();
}

}  // namespace nvfp4
