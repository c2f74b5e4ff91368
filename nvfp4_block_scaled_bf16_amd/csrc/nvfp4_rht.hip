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
// Two passes over x, like the ordinary per-token cast: the amax of the
// transformed columns, then the transform again with the encoding.  A lane
// holds a 16-row x 8-column sub-block (one 16-byte word per row); a
// workgroup of 4 waves covers 128 rows x 256 columns.  Requires M % 16 == 0
// and K % 8 == 0.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_device.hpp"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

constexpr int kRhtCols = 256;        // columns per workgroup (32 lanes x 8)
constexpr int kRhtRows = 128;        // rows per workgroup step (4 waves x 2 row groups x 16)
constexpr int kRhtAmaxSteps = 4;     // steps per workgroup in the amax pass (512 rows)

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

// the transformed column k of the lane's 16 x 8 sub-block: y[i] as fp32 bits
// of bf16 values
__device__ __forceinline__ void rht_column(const u32x4 (&v)[16], int k, uint32_t mask, uint32_t (&y)[16]) {
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) t[i] = __uint_as_float(col_bits(v[i], k) ^ (((mask >> i) & 1u) << 31));
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
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = round_to_bf16(t[i] * 0.25f);
}

__device__ __forceinline__ uint32_t mag16(uint32_t fbits) { return (fbits >> 16) & 0x7fffu; }

// Pass 1: the amax of the transformed tensor, per column (col_amax [K],
// zeroed beforehand) or for the whole tensor (col_amax [1]).  Grid:
// (cdiv(K, 256), cdiv(M, 512)).
template <int MODE>
__global__ __launch_bounds__(256) void k_rht_amax(const uint16_t* __restrict__ x, int64_t M, int64_t K, uint32_t mask,
                                                  float* __restrict__ col_amax) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, rg = lane >> 5;
    const int64_t c0 = (int64_t)blockIdx.x * kRhtCols + (lane & 31) * 8;
    const bool col_ok = c0 < K;
    uint32_t m[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll 1
    for (int step = 0; step < kRhtAmaxSteps; ++step) {
        const int64_t r0 = ((int64_t)blockIdx.y * kRhtAmaxSteps + step) * kRhtRows + wave * 32 + 16 * rg;
        if (!col_ok || r0 >= M) continue;   // M % 16 == 0: a row group is whole or absent
        u32x4 v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = *reinterpret_cast<const u32x4*>(x + (r0 + i) * K + c0);
        // columns unrolled: a column index that varies at run time would put
        // v in scratch memory
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            uint32_t y[16];
            rht_column(v, k, mask, y);
            uint32_t b = 0u;
#pragma unroll
            for (int i = 0; i < 16; ++i) b = b > mag16(y[i]) ? b : mag16(y[i]);
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
        // the workgroup's maximum, then one atomic
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const uint32_t o = (uint32_t)__shfl_xor((int)b, off);
            b = b > o ? b : o;
        }
        __shared__ uint32_t wred[4];
        if (lane == 0) wred[wave] = b;
        __syncthreads();
        if (t == 0) {
            b = wred[0];
            for (int w = 1; w < 4; ++w) b = b > wred[w] ? b : wred[w];
            if (b != 0u) atomicMax(reinterpret_cast<uint32_t*>(col_amax), b << 16);
        }
    }
}

// E2M1 codes of the 16 transformed values of one column block into two
// words (element i in nibble i % 8 of word i / 8), with the block's E4M3 code
struct ColCodes {
    uint32_t lo, hi, code;
};

__device__ __forceinline__ ColCodes encode_column(const uint32_t (&y)[16], float A) {
    uint32_t b = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) b = b > mag16(y[i]) ? b : mag16(y[i]);
    const Outer o = make_outer(A);
    const FastBlock fb = fast_block<false>(b << 16, o);
    ColCodes c{0u, 0u, 0u};
    if (__builtin_amdgcn_ballot_w64(o.slow || fb.slow) == 0ull) {
        float q[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) q[i] = quot2(__uint_as_float(y[i]), fb.yh, fb.yl);
        c.lo = put_fp4x2<0>(0u, q[0], q[1]);
        c.lo = put_fp4x2<1>(c.lo, q[2], q[3]);
        c.lo = put_fp4x2<2>(c.lo, q[4], q[5]);
        c.lo = put_fp4x2<3>(c.lo, q[6], q[7]);
        c.hi = put_fp4x2<0>(0u, q[8], q[9]);
        c.hi = put_fp4x2<1>(c.hi, q[10], q[11]);
        c.hi = put_fp4x2<2>(c.hi, q[12], q[13]);
        c.hi = put_fp4x2<3>(c.hi, q[14], q[15]);
        c.code = fb.code & 0xffu;
    } else {
        // exact path: IEEE block scale and element divisions
        const BlockScale bs = block_scale(b, outer_scale(A));
        float q[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float a = __uint_as_float(y[i]);
            q[i] = bs.zero ? a * 0.0f : a / bs.r;
        }
        c.lo = put_fp4x2<0>(0u, q[0], q[1]);
        c.lo = put_fp4x2<1>(c.lo, q[2], q[3]);
        c.lo = put_fp4x2<2>(c.lo, q[4], q[5]);
        c.lo = put_fp4x2<3>(c.lo, q[6], q[7]);
        c.hi = put_fp4x2<0>(0u, q[8], q[9]);
        c.hi = put_fp4x2<1>(c.hi, q[10], q[11]);
        c.hi = put_fp4x2<2>(c.hi, q[12], q[13]);
        c.hi = put_fp4x2<3>(c.hi, q[14], q[15]);
        c.code = bs.code;
    }
    return c;
}

// Pass 2: transform and encode.  col_q [K][M/2], col_sf [K][M/16].  Grid:
// (cdiv(K, 256), cdiv(M, 128)).
template <int MODE>
__global__ __launch_bounds__(256) void k_rht_encode(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                    uint32_t mask, const float* __restrict__ col_amax,
                                                    uint8_t* __restrict__ col_q, uint8_t* __restrict__ col_sf) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, rg = lane >> 5;
    const int64_t c0 = (int64_t)blockIdx.x * kRhtCols + (lane & 31) * 8;
    const int64_t r0 = (int64_t)blockIdx.y * kRhtRows + wave * 32 + 16 * rg;
    // M % 16 == 0: a row group is whole or absent; inactive lanes still take
    // part in the wave-wide path choice
    const bool active = c0 < K && r0 < M;
    u32x4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        v[i] = active ? *reinterpret_cast<const u32x4*>(x + (r0 + i) * K + c0) : u32x4{0u, 0u, 0u, 0u};
    const float At = MODE == ENC_TENSOR ? col_amax[0] : 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {   // unrolled (see k_rht_amax)
        uint32_t y[16];
        rht_column(v, k, mask, y);
        const float A = MODE == ENC_TENSOR ? At : (active ? col_amax[c0 + k] : 0.0f);
        const ColCodes c = encode_column(y, A);
        if (active) {
            *reinterpret_cast<u32x2*>(col_q + (c0 + k) * (M / 2) + r0 / 2) = u32x2{c.lo, c.hi};
            col_sf[(c0 + k) * (M / 16) + r0 / 16] = (uint8_t)c.code;
        }
    }
}

}  // namespace

hipError_t launch_rht_columnwise(int mode, const uint16_t* x, int64_t M, int64_t K, uint32_t mask, float* col_amax,
                                 uint8_t* col_q, uint8_t* col_sf, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    if (M <= 0 || K <= 0) return hipSuccess;
    const unsigned gx = (unsigned)((K + kRhtCols - 1) / kRhtCols);
    const dim3 ga(gx, (unsigned)((M + kRhtRows * kRhtAmaxSteps - 1) / (kRhtRows * kRhtAmaxSteps)));
    const dim3 ge(gx, (unsigned)((M + kRhtRows - 1) / kRhtRows));
    if (mode == ENC_TOKEN) {
        hipLaunchKernelGGL(k_rht_amax<ENC_TOKEN>, ga, dim3(256), 0, st, x, M, K, mask, col_amax);
        hipExtLaunchKernelGGL(k_rht_encode<ENC_TOKEN>, ge, dim3(256), 0, st, ev0, ev1, 0, x, M, K, mask,
                              (const float*)col_amax, col_q, col_sf);
    } else {
        hipLaunchKernelGGL(k_rht_amax<ENC_TENSOR>, ga, dim3(256), 0, st, x, M, K, mask, col_amax);
        hipExtLaunchKernelGGL(k_rht_encode<ENC_TENSOR>, ge, dim3(256), 0, st, ev0, ev1, 0, x, M, K, mask,
                              (const float*)col_amax, col_q, col_sf);
    }
    return hipGetLastError();
}

}  // namespace nvfp4
