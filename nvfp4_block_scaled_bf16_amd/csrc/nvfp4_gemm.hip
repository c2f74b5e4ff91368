// nvfp4_gemm.hip -- the NVFP4 GEMM consumer for gfx950: two NVFP4 operands
// with 16-element blocks along the contraction dimension K, rescaled by the
// per-row / per-column outer scales in the epilogue (the GEMM of the per-token
// recipe page, TransformerEngine PR #3045, "Changes" and the sequence
// diagram's TN forward product; its NN dgrad and NT wgrad products are this
// form applied to the cast's columnwise output):
//   out[m][n] = S_a(m) * S_b(n) * sum_k (g * D)_a[m][k] * (g * D)_b[n][k]
// with g the E2M1 value, D the decoded E4M3 block scale and S = amax / 2688.
//
// g * D has at most 6 significant bits, so it is exact in bf16: each K step
// dequantizes the operands' FP4 bytes into bf16 tiles in LDS and the
// contraction runs on bf16 MFMA (v_mfma_f32_32x32x16_bf16) with fp32
// accumulation; the outer scales multiply the accumulators in the epilogue.
// (gfx950's scaled FP4 MFMA takes one power-of-two scale per 32 elements and
// cannot carry an E4M3 scale per 16.)
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_device.hpp"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kTileM = 128, kTileN = 128;   // output tile per workgroup (4 waves, 2 x 2, 64 x 64 each)
constexpr int kStepK = 64;                  // K per pipeline step: 4 scale blocks
constexpr int kPitch = kStepK + 8;          // bf16 per LDS tile row (padding spreads the rows over the banks)

// E4M3 code -> value (exact): subnormals m * 2^-9, else exponent + 120 in fp32
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
    return code < 8u ? (float)code * 0.001953125f : __uint_as_float((code << 20) + 0x3C000000u);
}

// One thread's share of a K step for one operand: 32 consecutive elements
// (two scale blocks) of one row.  Rows past the end and blocks past K read
// as zeros.
struct RowPiece {
    uint32_t q[4];      // 16 bytes: 32 nibbles, element 2i in the low nibble
    uint32_t sf;        // two scale codes: low byte, next byte
};

__device__ __forceinline__ RowPiece load_piece(const uint8_t* __restrict__ q, const uint8_t* __restrict__ sf,
                                               int64_t row, int64_t rows, int64_t K, int64_t k0) {
    RowPiece p{{0u, 0u, 0u, 0u}, 0u};
    if (row < rows) {
        const uint8_t* qr = q + row * (K / 2);
        const uint8_t* sr = sf + row * (K / 16);
        if (k0 < K) {
            const uint2 lo = *reinterpret_cast<const uint2*>(qr + k0 / 2);
            p.q[0] = lo.x;
            p.q[1] = lo.y;
            p.sf = sr[k0 / 16];
        }
        if (k0 + 16 < K) {
            const uint2 hi = *reinterpret_cast<const uint2*>(qr + k0 / 2 + 8);
            p.q[2] = hi.x;
            p.q[3] = hi.y;
            p.sf |= (uint32_t)sr[k0 / 16 + 1] << 8;
        }
    }
    return p;
}

// dequantize a piece into 32 bf16 (g * D, exact) and store it to LDS
__device__ __forceinline__ void store_piece(const RowPiece& p, __bf16* dst) {
    const float d0 = e4m3_to_f32(p.sf & 0xffu), d1 = e4m3_to_f32(p.sf >> 8);
    bf16x8 out[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float d = w < 2 ? d0 : d1;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            // byte b of word w: elements 8w + 2b (low nibble) and 8w + 2b + 1;
            // the conversion with scale 1.0 gives the E2M1 values exactly
            f32x2 g;
            if (b == 0) g = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p.q[w], 1.0f, 0);
            else if (b == 1) g = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p.q[w], 1.0f, 1);
            else if (b == 2) g = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p.q[w], 1.0f, 2);
            else g = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p.q[w], 1.0f, 3);
            out[w][2 * b] = (__bf16)(g.x * d);
            out[w][2 * b + 1] = (__bf16)(g.y * d);
        }
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) *reinterpret_cast<bf16x8*>(dst + 8 * w) = out[w];
}

// Grid: cdiv(M, 128) * cdiv(N, 128) workgroups (one dimension), 256 threads;
// ntn = cdiv(N, 128).  Thread t loads row t / 2, elements 32 * (t % 2) .. + 31
// of each K step for both operands.
__global__ __launch_bounds__(256) void k_gemm_nvfp4(const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_sf,
                                                    const float* __restrict__ a_amax, int a_per_row,
                                                    const uint8_t* __restrict__ b_q, const uint8_t* __restrict__ b_sf,
                                                    const float* __restrict__ b_amax, int b_per_row,
                                                    int64_t M, int64_t N, int64_t K, uint32_t ntn,
                                                    float* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) __bf16 As[2][kTileM * kPitch];
    __shared__ __attribute__((aligned(16))) __bf16 Bs[2][kTileN * kPitch];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;   // the wave's 64 x 64 quarter
    // XCD-aware order: each of the 8 XCDs (own L2) takes a contiguous run of
    // tiles, row band major, so a band of A is reused from one L2
    const uint32_t ntiles = gridDim.x, lin = blockIdx.x;
    const uint32_t tile = (ntiles & 7u) == 0u ? (lin & 7u) * (ntiles >> 3) + (lin >> 3) : lin;
    const int64_t m0 = (int64_t)(tile / ntn) * kTileM, n0 = (int64_t)(tile % ntn) * kTileN;
    const int lr = t >> 1, lh = t & 1;   // load row, half

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    const int64_t nk = (K + kStepK - 1) / kStepK;
    RowPiece pa = load_piece(a_q, a_sf, m0 + lr, M, K, 32 * lh);
    RowPiece pb = load_piece(b_q, b_sf, n0 + lr, N, K, 32 * lh);
    store_piece(pa, &As[0][lr * kPitch + 32 * lh]);
    store_piece(pb, &Bs[0][lr * kPitch + 32 * lh]);
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int buf = (int)(kt & 1);
        const bool more = kt + 1 < nk;
        if (more) {   // the next step's bytes, in flight during this step's MFMAs
            pa = load_piece(a_q, a_sf, m0 + lr, M, K, (kt + 1) * kStepK + 32 * lh);
            pb = load_piece(b_q, b_sf, n0 + lr, N, K, (kt + 1) * kStepK + 32 * lh);
        }
        const __bf16* as = As[buf];
        const __bf16* bs = Bs[buf];
#pragma unroll
        for (int kc = 0; kc < kStepK / 16; ++kc) {
            const int kk = 16 * kc + 8 * (lane >> 5);
            bf16x8 fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                fa[i] = *reinterpret_cast<const bf16x8*>(as + (wm * 64 + 32 * i + (lane & 31)) * kPitch + kk);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                fb[j] = *reinterpret_cast<const bf16x8*>(bs + (wn * 64 + 32 * j + (lane & 31)) * kPitch + kk);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            store_piece(pa, &As[buf ^ 1][lr * kPitch + 32 * lh]);
            store_piece(pb, &Bs[buf ^ 1][lr * kPitch + 32 * lh]);
        }
        __syncthreads();
    }

    // epilogue: out = RN(RN(acc * S_a) * S_b); accumulator a of lane l holds
    // row 8 (a / 4) + 4 (l / 32) + a % 4, column l % 32 of its 32 x 32 block
    const float sa_t = a_per_row ? 0.0f : outer_scale(a_amax[0]);
    const float sb_t = b_per_row ? 0.0f : outer_scale(b_amax[0]);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t col = n0 + wn * 64 + 32 * j + (lane & 31);
        const bool col_ok = col < N;
        const float sb = b_per_row ? (col_ok ? outer_scale(b_amax[col]) : 0.0f) : sb_t;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int a = 0; a < 16; ++a) {
                const int64_t row = m0 + wm * 64 + 32 * i + 8 * (a >> 2) + 4 * (lane >> 5) + (a & 3);
                if (row < M && col_ok) {
                    const float sa = a_per_row ? outer_scale(a_amax[row]) : sa_t;
                    out[row * N + col] = (acc[i][j][a] * sa) * sb;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_nvfp4(const uint8_t* a_q, const uint8_t* a_sf, const float* a_amax, int a_per_row,
                             const uint8_t* b_q, const uint8_t* b_sf, const float* b_amax, int b_per_row,
                             int64_t M, int64_t N, int64_t K, float* out, hipStream_t st, hipEvent_t ev0,
                             hipEvent_t ev1) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const int64_t ntn = (N + kTileN - 1) / kTileN, ntiles = ntn * ((M + kTileM - 1) / kTileM);
    if (ntiles > kMaxGemmTiles) return hipErrorInvalidValue;
    hipExtLaunchKernelGGL(k_gemm_nvfp4, dim3((unsigned)ntiles), dim3(256), 0, st, ev0, ev1, 0, a_q, a_sf, a_amax,
                          a_per_row, b_q, b_sf, b_amax, b_per_row, M, N, K, (uint32_t)ntn, out);
    return hipGetLastError();
}

}  // namespace nvfp4
