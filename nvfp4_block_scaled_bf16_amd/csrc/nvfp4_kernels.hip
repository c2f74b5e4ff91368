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
constexpr int kEncRows = 64;       // rows per workgroup tile in the encode pass

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

// MODE: ENC_TENSOR (amax[0] for every vector), ENC_TOKEN (row_amax[r],
// col_amax[c]), ENC_TILE (16x16 tiles, tensor amax in row_amax[0]; also fills
// row_amax[1..M) and col_amax[1..K) with it), ENC_GROUPED (rowwise per-token;
// columnwise per expert with col_amax[e][K] and per-expert output slabs).
template <int MODE, bool ROW, bool COL>
__global__ __launch_bounds__(256) void k_encode(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                int64_t row_begin, int64_t row_end,
                                                const float* __restrict__ row_amax, const float* __restrict__ col_amax,
                                                uint8_t* __restrict__ row_q, uint8_t* __restrict__ row_sf,
                                                uint8_t* __restrict__ col_q, uint8_t* __restrict__ col_sf,
                                                float* __restrict__ fill_row, float* __restrict__ fill_col,
                                                GroupTable gt) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t c0 = (int64_t)blockIdx.x * kTileCols + lane * 8;
    const int64_t r0 = row_begin + (int64_t)blockIdx.y * kEncRows + wave * 16;
    const bool col_ok = c0 < K;
    if (MODE == ENC_TILE) {
        // broadcast the tensor amax into the per-token-layout vectors
        const float A = row_amax ? row_amax[0] : col_amax[0];
        const int64_t gid = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
        const int64_t gsz = (int64_t)gridDim.x * gridDim.y * blockDim.x;
        if (fill_row) for (int64_t i = 1 + gid; i < M; i += gsz) fill_row[i] = A;
        if (fill_col) for (int64_t i = 1 + gid; i < K; i += gsz) fill_col[i] = A;
    }
    if (r0 >= row_end || !col_ok) return;

    u32x4 v[16];
    load_subblock(x, K, r0, row_end, c0, true, v);

    // per-tensor outer scales (the split encode may carry different rowwise
    // and columnwise amax values); 16x16 tiles use the single tensor amax
    float S_row = 0.0f, S_col = 0.0f, S_tensor = 0.0f;
    if (MODE == ENC_TENSOR) {
        if (ROW) S_row = outer_scale(row_amax[0]);
        if (COL) S_col = outer_scale(col_amax[0]);
    }
    if (MODE == ENC_TILE) S_tensor = outer_scale(row_amax ? row_amax[0] : col_amax[0]);

    // 16x16 tile: one scale from the max over the tile (this lane's 16x8 half
    // and the neighbour's)
    BlockScale tile_bs;
    if (MODE == ENC_TILE) {
        uint32_t a = 0u;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            a = pk_max_u16(a, pk_max_u16(pk_max_u16(abs2(v[i].x), abs2(v[i].y)), pk_max_u16(abs2(v[i].z), abs2(v[i].w))));
        uint32_t m = max_halves(a);
        uint32_t o = (uint32_t)__shfl_xor((int)m, 1);
        tile_bs = block_scale(m > o ? m : o, S_tensor);
    }

    if (ROW) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t r = r0 + i;
            uint32_t a = pk_max_u16(pk_max_u16(abs2(v[i].x), abs2(v[i].y)), pk_max_u16(abs2(v[i].z), abs2(v[i].w)));
            uint32_t hm = max_halves(a);
            uint32_t other = (uint32_t)__shfl_xor((int)hm, 1);
            if (r >= row_end) continue;
            BlockScale bs;
            if (MODE == ENC_TILE) {
                bs = tile_bs;
            } else {
                float S = (MODE == ENC_TENSOR) ? S_row : outer_scale(row_amax[r]);
                bs = block_scale(hm > other ? hm : other, S);
            }
            uint32_t packed = encode8(v[i], bs);
            *reinterpret_cast<uint32_t*>(row_q + r * (K / 2) + c0 / 2) = packed;
            if ((lane & 1) == 0) row_sf[r * (K / 16) + c0 / 16] = (uint8_t)bs.code;
        }
    }

    if (COL) {
        // column maxima over the 16 rows, packed pairs of columns
        uint32_t cm[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            cm[0] = pk_max_u16(cm[0], abs2(v[i].x));
            cm[1] = pk_max_u16(cm[1], abs2(v[i].y));
            cm[2] = pk_max_u16(cm[2], abs2(v[i].z));
            cm[3] = pk_max_u16(cm[3], abs2(v[i].w));
        }
        // where this sub-block's columnwise output goes
        int64_t m_len = M, row0 = 0, amax_row = 0;
        if (MODE == ENC_GROUPED) {
            int g = group_of_row(gt, r0);
            m_len = gt.cnt[g];
            row0 = gt.off[g];
            amax_row = (int64_t)(gt.first + g) * K;
        }
        uint8_t* qbase = col_q + row0 * K / 2;
        uint8_t* sbase = col_sf + row0 * K / 16;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t c = c0 + j;
            const uint32_t w = cm[j >> 1];
            const uint32_t bmag = (j & 1) ? (w >> 16) : (w & 0xffffu);
            BlockScale bs;
            if (MODE == ENC_TILE) {
                bs = tile_bs;
            } else {
                float S = (MODE == ENC_TENSOR) ? S_col : outer_scale(col_amax[amax_row + c]);
                bs = block_scale(bmag, S);
            }
            float e[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                uint32_t word = (j >> 1) == 0 ? v[i].x : (j >> 1) == 1 ? v[i].y : (j >> 1) == 2 ? v[i].z : v[i].w;
                e[i] = (j & 1) ? bf_hi(word) : bf_lo(word);
            }
            uint32_t lo = 0u, hi = 0u;
            lo = put_fp4x2<0>(lo, quotient(e[0], bs), quotient(e[1], bs));
            lo = put_fp4x2<1>(lo, quotient(e[2], bs), quotient(e[3], bs));
            lo = put_fp4x2<2>(lo, quotient(e[4], bs), quotient(e[5], bs));
            lo = put_fp4x2<3>(lo, quotient(e[6], bs), quotient(e[7], bs));
            hi = put_fp4x2<0>(hi, quotient(e[8], bs), quotient(e[9], bs));
            hi = put_fp4x2<1>(hi, quotient(e[10], bs), quotient(e[11], bs));
            hi = put_fp4x2<2>(hi, quotient(e[12], bs), quotient(e[13], bs));
            hi = put_fp4x2<3>(hi, quotient(e[14], bs), quotient(e[15], bs));
            *reinterpret_cast<u32x2*>(qbase + c * (m_len / 2) + (r0 - row0) / 2) = u32x2{lo, hi};
            sbase[c * (m_len / 16) + (r0 - row0) / 16] = (uint8_t)bs.code;
        }
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

template <int MODE>
static void launch_encode_mode(bool row, bool col, dim3 grid, hipStream_t st, const uint16_t* x, int64_t M, int64_t K,
                               int64_t rb, int64_t re, const float* ra, const float* ca, uint8_t* rq, uint8_t* rs,
                               uint8_t* cq, uint8_t* cs, float* fr, float* fc, const GroupTable& gt) {
    if (row && col)
        hipLaunchKernelGGL((k_encode<MODE, true, true>), grid, dim3(256), 0, st, x, M, K, rb, re, ra, ca, rq, rs, cq, cs, fr, fc, gt);
    else if (row)
        hipLaunchKernelGGL((k_encode<MODE, true, false>), grid, dim3(256), 0, st, x, M, K, rb, re, ra, ca, rq, rs, cq, cs, fr, fc, gt);
    else
        hipLaunchKernelGGL((k_encode<MODE, false, true>), grid, dim3(256), 0, st, x, M, K, rb, re, ra, ca, rq, rs, cq, cs, fr, fc, gt);
}

hipError_t launch_encode(int mode, bool row, bool col, const uint16_t* x, int64_t M, int64_t K,
                         int64_t row_begin, int64_t row_end, const float* row_amax, const float* col_amax,
                         uint8_t* row_q, uint8_t* row_sf, uint8_t* col_q, uint8_t* col_sf,
                         float* fill_row, float* fill_col, const GroupTable& gt, hipStream_t st) {
    if (row_end <= row_begin || K <= 0 || (!row && !col)) return hipSuccess;
    dim3 grid(cdiv(K, kTileCols), cdiv(row_end - row_begin, kEncRows));
    switch (mode) {
    case ENC_TENSOR:
        launch_encode_mode<ENC_TENSOR>(row, col, grid, st, x, M, K, row_begin, row_end, row_amax, col_amax, row_q, row_sf, col_q, col_sf, fill_row, fill_col, gt);
        break;
    case ENC_TOKEN:
        launch_encode_mode<ENC_TOKEN>(row, col, grid, st, x, M, K, row_begin, row_end, row_amax, col_amax, row_q, row_sf, col_q, col_sf, fill_row, fill_col, gt);
        break;
    case ENC_TILE:
        launch_encode_mode<ENC_TILE>(row, col, grid, st, x, M, K, row_begin, row_end, row_amax, col_amax, row_q, row_sf, col_q, col_sf, fill_row, fill_col, gt);
        break;
    default:
        launch_encode_mode<ENC_GROUPED>(row, col, grid, st, x, M, K, row_begin, row_end, row_amax, col_amax, row_q, row_sf, col_q, col_sf, fill_row, fill_col, gt);
        break;
    }
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
