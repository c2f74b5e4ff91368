// nvfp4_rows.hip -- the single-pass per-token rowwise cast for gfx950.
//
// Per-token scaling gives every row its own outer amax (TransformerEngine PR
// #3045, "Add NVFP4 per-token quantization recipe", Description: a per-row
// amax vector of length M for rowwise data), so a workgroup that owns whole
// rows can reduce each row's amax on chip and encode the row from the same
// registers: x is read once.  k_rows does this for every rowwise-only
// per-token cast (plain and grouped).
//
// Decomposition: a workgroup is 8 waves (512 lanes); lane t holds columns
// 8t .. 8t+7 of every 4096-column round of a row, one 16-byte load per row
// and round.  A batch is R = L / NR rows of NR rounds (K <= 4096 NR), so a
// lane holds L loads (8, or 16 for 16 rounds).  A rowwise block (16 columns)
// is the lane pair (2j, 2j+1) at one load; the even lane computes the block
// parameters of the pair's even-numbered loads, the odd lane those of the
// odd-numbered ones, and DPP hands them across.  Row maxima: lane, then wave
// (xor exchanges), then the 8 waves through LDS (one barrier per batch); the
// row scales reach the other lanes by readlane.  Workgroup g takes batches
// g, g + G, ... and loads the next batch's rows while it encodes the current
// one (the host launches one workgroup per batch unless there are more than
// 2^20 batches, so that the dispatcher balances the load).  x is read with the nontemporal hint:
// nothing in the cast reads it again.
#include <hip/hip_ext.h>

#include "nvfp4_device.hpp"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr int kRowsWaves = 8;
constexpr int kRowsThreads = 64 * kRowsWaves;
constexpr int kRoundCols = 8 * kRowsThreads;   // 4096 columns per round
// 16-byte loads per lane per batch: 8 (72 VGPRs, up to three workgroups per
// CU), or 16 when a row has 16 rounds (a batch is at least one row)
constexpr int rows_loads(int nr) { return nr > 8 ? nr : 8; }

// elementwise max of packed 16-bit magnitudes over the wave (xor exchanges)
__device__ __forceinline__ uint32_t wave_max_pk(uint32_t v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = pk_max_u16(v, (uint32_t)__shfl_xor((int)v, d));
    return v;
}

// Exact re-encode of the blocks flagged in `mask` (bit f: load f of the
// batch; both lanes of a pair carry the pair's bits), with IEEE divisions,
// over what the fast path stored.  Data re-read from x; Av: lane r holds the
// amax of the batch's row r.  Inlined (a call inside the batch loop would
// have to preserve the next batch's data registers across it); the loop
// stays rolled.
template <int NR, int L>
__device__ __forceinline__ void rows_exact(const uint16_t* __restrict__ x, int64_t K, int64_t row0, uint32_t nrows,
                                        uint32_t mask, float Av, uint8_t* __restrict__ row_q,
                                        uint8_t* __restrict__ row_sf) {
    const uint32_t t = threadIdx.x;
#pragma unroll 1
    for (int f = 0; f < L; ++f) {
        if (!((mask >> f) & 1u)) continue;
        const int r = f / NR, n = f % NR;
        const int64_t col = (int64_t)n * kRoundCols + 8 * (int64_t)t;
        const bool in = (uint32_t)r < nrows && col < K;
        const int64_t row = row0 + r;
        const u32x4 w = in ? *reinterpret_cast<const u32x4*>(x + row * K + col) : u32x4{0u, 0u, 0u, 0u};
        uint32_t m = rowmax_word(w);
        m = pk_max_u16(m, from_pair(m));
        const float A = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Av), r));
        const BlockScale bs = block_scale(max_halves(m), outer_scale(A));
        uint32_t word = 0u;
#pragma unroll
        for (int k = 0; k < 8; k += 2) {
            const uint32_t h = k == 0 ? w.x : k == 2 ? w.y : k == 4 ? w.z : w.w;
            const float a0 = bf_lo(h), a1 = bf_hi(h);
            const float q0 = bs.zero ? a0 * 0.0f : a0 / bs.r, q1 = bs.zero ? a1 * 0.0f : a1 / bs.r;
            word |= (__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q0, q1, 1.0f, 0) & 0xffu) << (4 * k);
        }
        if (in) {
            *reinterpret_cast<uint32_t*>(row_q + row * (K / 2) + col / 2) = word;
            if (!(t & 1u)) row_sf[row * (K / 16) + col / 16] = (uint8_t)bs.code;
        }
    }
}

}  // namespace

// Rowwise per-token cast of rows [0, M): row_q [M][K/2], row_sf [M][K/16],
// row_amax [M] written here (no prior fill).  NR: 4096-column rounds per row
// (K <= 4096 NR, K % 16 == 0); FULL: K == 4096 NR, so that every round is
// whole and a lane's offsets differ between rounds by a constant (kept in
// the scalar offset).  L: loads per lane per batch.  nbatches = ceil(M / R);
// gridDim.x <= nbatches.
template <int NR, bool FULL, int L>
__global__ __launch_bounds__(kRowsThreads, L == 8 ? 5 : 4) void k_rows(const uint16_t* __restrict__ x, int64_t M,
                                                                        int64_t K, uint8_t* __restrict__ row_q,
                                                                        uint8_t* __restrict__ row_sf,
                                                                        float* __restrict__ row_amax, int64_t nbatches) {
    constexpr int R = L / NR;
    constexpr int RP = (R + 1) / 2;                   // packed row pairs
    __shared__ uint32_t red[2][kRowsWaves][RP];       // per batch parity: each wave's row maxima, two per word
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t t = threadIdx.x;
    const bool odd = lane & 1;
    const uint32_t xrow = (uint32_t)K * 2u, qrow = (uint32_t)(K / 2), srow = (uint32_t)(K / 16);

    // lane offsets of round n: voffset part (kOffOut past the last column:
    // loads read zeros, stores are dropped) and scalar part
    constexpr int NO = FULL ? 1 : NR;
    uint32_t xo[NO], qo[NO], so[NO];
#pragma unroll
    for (int n = 0; n < NO; ++n) {
        const int64_t col = (int64_t)n * kRoundCols + 8 * (int64_t)t;
        const bool ok = col < K;
        xo[n] = ok ? (uint32_t)col * 2u : kOffOut;
        qo[n] = ok ? (uint32_t)(col / 2) : kOffOut;
        so[n] = ok ? (uint32_t)(col / 16) : kOffOut;
    }
    auto xv = [&](int n) { return FULL ? xo[0] : xo[n]; };
    auto qv = [&](int n) { return FULL ? qo[0] : qo[n]; };
    auto sv = [&](int n) { return FULL ? so[0] : so[n]; };
    auto xs = [&](int n) { return FULL ? (uint32_t)n * (2u * kRoundCols) : 0u; };
    auto qs = [&](int n) { return FULL ? (uint32_t)n * (kRoundCols / 2u) : 0u; };
    auto ss = [&](int n) { return FULL ? (uint32_t)n * (kRoundCols / 16u) : 0u; };
    auto batch_rows = [&](int64_t b) -> uint32_t {
        const int64_t left = M - b * R;
        return left <= 0 ? 0u : (left < R ? (uint32_t)left : (uint32_t)R);
    };
    // the row stride is opaque to keep per-row offsets in scalar registers
    uint32_t xr = xrow;
    asm volatile("" : "+s"(xr));

    int64_t b = blockIdx.x;
    u32x4 v[L];
    {
        const __amdgpu_buffer_rsrc_t rs = rsrc(x + b * R * K, batch_rows(b) * xrow);
#pragma unroll
        for (int f = 0; f < L; ++f)
            v[f] = __builtin_amdgcn_raw_buffer_load_b128(rs, xv(f % NR), (f / NR) * xr + xs(f % NR), kCacheNT);
    }
    int par = 0;
#pragma unroll 1
    for (; b < nbatches; b += gridDim.x, par ^= 1) {
        const int64_t row0 = b * R;
        const uint32_t nrows = batch_rows(b);
        const int64_t bn = b + gridDim.x;
        const __amdgpu_buffer_rsrc_t nrs = bn < nbatches ? rsrc(x + bn * R * K, batch_rows(bn) * xrow) : rsrc(x, 0u);

        // (1) maxima: per load the lane's (even, odd) column maxima, per row
        // the wave's maximum, per pair of loads the two blocks' maxima
        uint32_t bm[L / 2];
        {
            uint32_t rw[L];
#pragma unroll
            for (int f = 0; f < L; ++f) {
                const uint32_t a0 = abs2(v[f].x), a1 = abs2(v[f].y), a2 = abs2(v[f].z), a3 = abs2(v[f].w);
                rw[f] = pk_max_u16(pk_max_u16(a0, a1), pk_max_u16(a2, a3));
            }
#pragma unroll
            for (int p = 0; p < RP; ++p) {
                uint32_t lo = 0u, hi = 0u;
#pragma unroll
                for (int n = 0; n < NR; ++n) {
                    lo = pk_max_u16(lo, rw[(2 * p) * NR + n]);
                    if (2 * p + 1 < R) hi = pk_max_u16(hi, rw[(2 * p + 1) * NR + n]);
                }
                const uint32_t m = wave_max_pk(max_halves(lo) | (max_halves(hi) << 16));
                if (lane == 0) red[par][wave][p] = m;
            }
            // own half of the pair's maximum moved to the top: fp32 bits
            const uint32_t own_sel = odd ? 0x03020c0cu : 0x01000c0cu;
#pragma unroll
            for (int k = 0; k < L / 2; ++k) {
                uint32_t m = pk_max_u16(__builtin_amdgcn_perm(rw[2 * k + 1], rw[2 * k], 0x05040100u),
                                        __builtin_amdgcn_perm(rw[2 * k + 1], rw[2 * k], 0x07060302u));
                m = pk_max_u16(m, from_pair(m));
                bm[k] = __builtin_amdgcn_perm(m, m, own_sel);
            }
        }
#pragma unroll
        for (int k = 0; k < L / 2; ++k) asm volatile("" : "+v"(bm[k]));
        __syncthreads();

        // (2) row amax over the waves: lane r < R takes row r and its outer
        // scale; the other lanes take them with readlane (wave 0 writes
        // row_amax)
        const int rl = lane < R ? lane : 0;
        float Av;
        Outer ov;
        {
            uint32_t m = 0u;
#pragma unroll
            for (int w = 0; w < kRowsWaves; ++w) m = pk_max_u16(m, red[par][w][rl >> 1]);
            Av = mag_to_f32((rl & 1) ? (m >> 16) : (m & 0xffffu));
            ov = make_outer(Av);
            if (wave == 0 && lane < R && (uint32_t)lane < nrows) row_amax[row0 + lane] = Av;
        }
        const uint64_t oslow = __builtin_amdgcn_ballot_w64(lane < R && ov.slow);
        auto lane_f = [](float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); };

        // (3) per pair of loads: block parameters of the lane's own load
        // (2k even lane, 2k+1 odd lane), its scale byte, then both loads
        // encoded, stored, and the next batch's rows loaded in their place
        const __amdgpu_buffer_rsrc_t q_rs = rsrc(row_q + row0 * (K / 2), nrows * qrow);
        const __amdgpu_buffer_rsrc_t s_rs = rsrc(row_sf + row0 * (K / 16), nrows * srow);
        uint32_t slow = 0u;
#pragma unroll
        for (int k = 0; k < L / 2; ++k) {
            const int fe = 2 * k, fo = 2 * k + 1;
            const int rown = odd ? fo / NR : fe / NR;        // row of the own block
            Outer o;
            if (fe / NR == fo / NR) {
                o.S = lane_f(ov.S, fe / NR);
                o.yS = lane_f(ov.yS, fe / NR);
            } else {
                o.S = odd ? lane_f(ov.S, fo / NR) : lane_f(ov.S, fe / NR);
                o.yS = odd ? lane_f(ov.yS, fo / NR) : lane_f(ov.yS, fe / NR);
            }
            const FastBlock fb = fast_block<false, true>(bm[k], o);
            const bool bslow = fb.slow || ((oslow >> rown) & 1ull);
            slow |= (bslow ? 1u : 0u) << (odd ? fo : fe);
            const uint32_t vo = odd ? sv(fo % NR) + ss(fo % NR) + (uint32_t)(fo / NR) * srow
                                    : sv(fe % NR) + ss(fe % NR) + (uint32_t)(fe / NR) * srow;
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)fb.code, s_rs, vo, 0, 0);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int f = 2 * k + h;
                const float bh = h ? from_odd(fb.yh) : from_even(fb.yh);
                const float bl = h ? from_odd(fb.yl) : from_even(fb.yl);
                const u32x4 w = v[f];
                const float q0 = quot2(bf_lo(w.x), bh, bl);
                uint32_t o4 = put_fp4x2<0>(__float_as_uint(q0), q0, quot2(bf_hi(w.x), bh, bl));
                o4 = put_fp4x2<1>(o4, quot2(bf_lo(w.y), bh, bl), quot2(bf_hi(w.y), bh, bl));
                o4 = put_fp4x2<2>(o4, quot2(bf_lo(w.z), bh, bl), quot2(bf_hi(w.z), bh, bl));
                o4 = put_fp4x2<3>(o4, quot2(bf_lo(w.w), bh, bl), quot2(bf_hi(w.w), bh, bl));
                __builtin_amdgcn_raw_buffer_store_b32(o4, q_rs, qv(f % NR), (uint32_t)(f / NR) * qrow + qs(f % NR),
                                                      kCacheNT);
                // the next batch's load f, issued once this word is done
                uint32_t xsf = (uint32_t)(f / NR) * xr + xs(f % NR);
                asm volatile("" : "+s"(xsf) : "v"(o4));
                v[f] = __builtin_amdgcn_raw_buffer_load_b128(nrs, xv(f % NR), xsf, kCacheNT);
            }
        }

        // (4) blocks outside the fast path's range: exact, over what was stored
        const uint32_t mask = slow | from_pair(slow);
        if (__builtin_amdgcn_ballot_w64(mask != 0u) != 0ull)
            rows_exact<NR, L>(x, K, row0, nrows, mask, Av, row_q, row_sf);
    }

}

// rounds per row for K, or 0 when K is beyond the single-pass kernel
int rows_rounds(int64_t K) {
    const int64_t n = (K + kRoundCols - 1) / kRoundCols;
    return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : n <= 8 ? 8 : n <= 16 ? 16 : 0;
}

int64_t rows_batches(int64_t M, int64_t K) {
    const int nr = rows_rounds(K);
    if (nr == 0) return 0;
    const int rows = rows_loads(nr) / nr;
    return (M + rows - 1) / rows;
}

template <int NR>
static void launch_rows_nr(unsigned grid, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1, const uint16_t* x, int64_t M,
                           int64_t K, uint8_t* q, uint8_t* sf, float* amax, int64_t nb) {
    constexpr int L = rows_loads(NR);
    if (K == (int64_t)NR * kRoundCols)
        hipExtLaunchKernelGGL((k_rows<NR, true, L>), dim3(grid), dim3(kRowsThreads), 0, st, ev0, ev1, 0, x, M, K, q, sf,
                              amax, nb);
    else
        hipExtLaunchKernelGGL((k_rows<NR, false, L>), dim3(grid), dim3(kRowsThreads), 0, st, ev0, ev1, 0, x, M, K, q,
                              sf, amax, nb);
}

hipError_t launch_rows(const uint16_t* x, int64_t M, int64_t K, uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                       unsigned grid, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    const int nr = rows_rounds(K);
    const int64_t nb = rows_batches(M, K);
    if (nr == 0 || M <= 0 || K <= 0 || grid == 0 || (int64_t)grid > nb) return hipErrorInvalidValue;
    switch (nr) {
    case 1: launch_rows_nr<1>(grid, st, ev0, ev1, x, M, K, row_q, row_sf, row_amax, nb); break;
    case 2: launch_rows_nr<2>(grid, st, ev0, ev1, x, M, K, row_q, row_sf, row_amax, nb); break;
    case 4: launch_rows_nr<4>(grid, st, ev0, ev1, x, M, K, row_q, row_sf, row_amax, nb); break;
    case 8: launch_rows_nr<8>(grid, st, ev0, ev1, x, M, K, row_q, row_sf, row_amax, nb); break;
    default: launch_rows_nr<16>(grid, st, ev0, ev1, x, M, K, row_q, row_sf, row_amax, nb); break;
    }
    return hipGetLastError();
}

}  // namespace nvfp4
