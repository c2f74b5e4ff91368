// nvfp4_kernels.hip -- HIP kernels of the bf16 -> NVFP4 cast for gfx950:
// outer amax, encode (rowwise and columnwise from one read), 16x16 tiles,
// grouped experts, dequantize and the decayed accumulator.  They serve every
// shape the C ABI accepts.
//
// Work decomposition shared by the amax and encode kernels: a lane owns a
// 16-row x 8-column sub-block (sixteen 16-byte loads, one per row), so one
// load instruction reads 16 bytes per lane along a row (1 KB of one row per
// wave in the amax pass; 512 bytes of each of two rows in the encode pass,
// whose waves are two 32-lane row groups).  A lane's 8 columns x 16 rows are
// eight complete columnwise blocks; the 16 rows hold half of a rowwise block
// each, the other half sitting in the neighbouring lane (lanes 2j and 2j+1
// exchange maxima and block parameters).
#include <hip/hip_ext.h>

#include "nvfp4_device.hpp"
#include "nvfp4_internal.h"

namespace nvfp4 {

constexpr int kTileCols = 512;     // columns per workgroup tile (64 lanes x 8)
constexpr int kAmaxRows = 512;     // rows per workgroup tile in the amax pass (at most; fewer for small tensors)
constexpr int kAmaxGroupedRows = 512;   // at most, for grouped casts (their per-expert LDS slots scale with it:
                                         // 32 slots x 512 columns, 64 KB)
constexpr int kEncRows = 256;      // rows per workgroup tile in the encode pass (at most; 128 for small tensors)
constexpr int kEncCols = 256;      // columns per workgroup tile in the encode pass: a wave is
                                   // two row groups of 32 lanes, each 16 rows x 256 columns
// LDS staging of a workgroup's columnwise output: per column, kEncRows rows
// give kEncRows/2 bytes of data and kEncRows/16 scale bytes; padded pitches
// spread the lanes' writes over the banks
constexpr int kStageQPitch = kEncRows / 2 + 4;
constexpr int kStageSfPitch = kEncRows / 16 + 4;
// longest run of 256-row tiles per workgroup in the resident cast
constexpr int kResMaxRun = 32;

// --------------------------------------------------------------- utilities

// fill two arrays (either may be empty) in one launch
__global__ void k_fill2_u32(uint32_t* __restrict__ p, int64_t n, uint32_t* __restrict__ q, int64_t m, uint32_t v) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t s = (int64_t)gridDim.x * blockDim.x;
    for (; i < n + m; i += s) {
        if (i < n) p[i] = v;
        else q[i - n] = v;
    }
}

// ------------------------------------------------ cross-workgroup waits
//
// One workgroup's writes sometimes have to reach the others before they go
// on: the amax pass zeroes its outputs in its first workgroups (the first
// dispatched) while the others will combine into them with atomics.  Such a
// launch gets a slot of g_sync_count (the count when it starts comes from
// the host): a workgroup arrives by adding 1 with release semantics (its
// writes reach memory first), and waits, one lane polling, until the slot
// reaches base + n.  The poll carries no acquire fence (on this chip an
// agent-scope acquire invalidates the caches, and one per wave costs more
// than a separate launch), so what a waiter does next must not read through
// the caches: device-scope atomics, which are performed beyond them, or
// loads that bypass them.  Every wait is bounded: after kSyncWaitTicks of
// the 100 MHz real-time clock it gives up, records the failure in the error
// word (host memory the library checks at its next call) and returns false,
// and the workgroup skips what depended on it.
constexpr uint64_t kSyncWaitTicks = 20000000ull;   // 0.2 s
__device__ unsigned long long g_sync_count[kSyncSlots];

__device__ __forceinline__ void sync_arrive(const SyncArg& s) {
    __hip_atomic_fetch_add(&g_sync_count[s.slot], 1ull, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// arrival for a workgroup whose prior writes are device-scope atomics or
// stores already complete (s_waitcnt): no cache write-back is needed
__device__ __forceinline__ void sync_arrive_relaxed(const SyncArg& s) {
    __hip_atomic_fetch_add(&g_sync_count[s.slot], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Grid-wide wait of a resident launch (one lane per workgroup): arrive with
// a fetch-and-add; the workgroup whose arrival is the last (the count it
// returns is base + n - 1) publishes base + n to kFlagLines flag words, one
// per 128-byte line, and goes on; every other workgroup polls the flag of
// line lin % kFlagLines.  All workgroups polling the arrival counter itself
// keep that one address busy at the memory side and delay the arrivals they
// wait for; spread over the lines, the wait passes about 4.5 us sooner.  The
// flags only grow (each launch on a slot publishes a larger count than the
// one before), so they are never cleared.  Bounded as sync_poll.
constexpr int kFlagLines = 16;
__device__ unsigned long long g_sync_flag[kSyncSlots][kFlagLines][16];

__device__ __forceinline__ bool sync_grid_wait(const SyncArg& s, unsigned long long n, uint32_t lin) {
    const unsigned long long target = s.base + n;
    const unsigned long long old =
        __hip_atomic_fetch_add(&g_sync_count[s.slot], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1ull == target) {
        for (int i = 0; i < kFlagLines; ++i)
            __hip_atomic_store(&g_sync_flag[s.slot][i][0], target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return true;
    }
    unsigned long long* f = &g_sync_flag[s.slot][lin % kFlagLines][0];
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
        if (__builtin_amdgcn_s_memrealtime() - t0 > kSyncWaitTicks) {
            __hip_atomic_store(s.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            return false;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    return true;
}

// one lane: wait for base + n arrivals; false when the wait gave up
__device__ __forceinline__ bool sync_poll(const SyncArg& s, unsigned long long n) {
    const unsigned long long target = s.base + n;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__hip_atomic_load(&g_sync_count[s.slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
        if (__builtin_amdgcn_s_memrealtime() - t0 > kSyncWaitTicks) {
            __hip_atomic_store(s.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            return false;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    return true;
}

// max of non-negative floats through their bit patterns
__device__ __forceinline__ void atomic_max_mag(float* p, uint32_t mag16) {
    if (mag16 != 0u) atomicMax(reinterpret_cast<uint32_t*>(p), mag16 << 16);
}

// load 16 rows x 8 bf16 (one 16-byte word per row) of a lane's sub-block;
// rows at or beyond row_end, and lanes past the last column (lane_off ==
// kOffOut), read zeros.  lane_off: the lane's byte offset within a row; xr:
// the row stride in bytes.  Ordinary (cached) loads: the amax pass leaves
// part of x in the last-level cache for the encode pass that follows, which
// measurably shortens it (nontemporal loads here make the amax pass a few
// microseconds faster and the encode pass more than that slower).
__device__ __forceinline__ void load_subblock(const uint16_t* __restrict__ x, int64_t K, int64_t r0,
                                              int64_t row_end, uint32_t lane_off, uint32_t xr, u32x4 v[16]) {
    const uint32_t nrows = (uint32_t)(row_end - r0 < 16 ? row_end - r0 : 16);
    const __amdgpu_buffer_rsrc_t rs = rsrc(x + r0 * K, nrows * xr);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane_off, i * xr, 0);
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
                                              float* __restrict__ t0, float* __restrict__ t1, GroupTable gt,
                                              int tile_h, ZeroFirst zero, SyncArg sync) {
    __shared__ uint32_t red[4][64][4];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar expert lookups
    // tile order: each XCD takes a contiguous run of tiles (row band major),
    // the order the encode pass walks too
    const uint32_t ntiles = gridDim.x * gridDim.y;
    const uint32_t lin = blockIdx.y * gridDim.x + blockIdx.x;
    const uint32_t tile = ((ntiles & 7u) == 0u) ? (lin & 7u) * (ntiles >> 3) + (lin >> 3) : lin;
    const uint32_t bx = tile % gridDim.x, by = tile / gridDim.x;
    const int64_t c0 = (int64_t)bx * kTileCols + lane * 8;
    const bool col_ok = c0 < K;
    // Zero-first: the first zero.wgs workgroups (dispatched first) clear the
    // outputs, kZeroPerWg values each, and arrive.  Every atomic of a
    // workgroup comes after its loop, behind one wait for those arrivals (one
    // lane polls, normally long satisfied); a wait that gave up skips the
    // atomics.
    const bool sync_on = sync.slot >= 0;
    if (sync_on && lin < (uint32_t)zero.wgs) {
        const int64_t z0 = (int64_t)lin * kZeroPerWg, z1 = z0 + kZeroPerWg;
        for (int64_t i = z0 + threadIdx.x; i < z1 && i < zero.na + zero.nb; i += blockDim.x) {
            if (i < zero.na) zero.a[i] = 0.0f;
            else zero.b[i - zero.na] = 0.0f;
        }
        __syncthreads();
        if (threadIdx.x == 0) sync_arrive(sync);
    }
    // one lane's wait for the zeroing workgroups (true: the outputs hold zeros)
    auto zeroed = [&]() -> bool { return !sync_on || sync_poll(sync, (unsigned long long)zero.wgs); };
    __shared__ int zero_ok;
    // Rows of the workgroup (tile_h: 64 to 512).  Per token, the four row
    // tiles of a group (by / 4, one strip) share the group's rows so that,
    // together, they read it from the top down in stripes of 256 rows, the
    // way the encode pass then walks it: workgroup k = by % 4, wave w, step j
    // take rows 16 (16 j + 4 w + k) .. + 15 of the group (measured faster
    // than one contiguous tile per workgroup, with the encode pass after
    // it).  Other kinds, and a group that is not four whole tiles, keep one
    // contiguous tile per workgroup (wave w: rows w tile_h / 4 ..).
    const int64_t grp0 = row_begin + (int64_t)(by & ~3u) * tile_h;
    const bool spread = KIND == AMAX_TOKEN && (by | 3u) < gridDim.y && grp0 + 4 * (int64_t)tile_h <= row_end;
    const int64_t rstride = spread ? 256 : 16;   // rows from one step of a wave to its next
    auto wave_row0 = [&](int w) -> int64_t {
        return spread ? grp0 + 16 * (4 * w + (int)(by & 3u)) : row_begin + (int64_t)by * tile_h + w * (tile_h / 4);
    };
    const int64_t rb = wave_row0(wave);
    const uint32_t lane_off = col_ok ? (uint32_t)c0 * 2u : kOffOut;
    uint32_t xr = (uint32_t)K * 2u;
    asm volatile("" : "+s"(xr));   // keeps the 16 row offsets from being held in registers
    uint32_t cm[4] = {0u, 0u, 0u, 0u};
    uint32_t tm = 0u;
    int cur_group = -1;
    // Grouped: column maxima are first combined in LDS per expert present
    // in the tile (slot = the expert's first row within the tile / 16, so at
    // most kAmaxGroupedRows / 16 slots), then one atomic per column and expert.
    constexpr int kSlots = kAmaxGroupedRows / 16;
    __shared__ uint32_t gred[KIND == AMAX_GROUPED ? kSlots : 1][KIND == AMAX_GROUPED ? kTileCols : 1];
    __shared__ int gslot[KIND == AMAX_GROUPED ? kSlots : 1];
    const int64_t tile_r0 = row_begin + (int64_t)by * tile_h;
    // the slots the tile's experts take (the experts overlapping a tile are
    // consecutive table entries): only those are cleared and combined
    uint32_t used = 0u;
    if (KIND == AMAX_GROUPED) {
        const int64_t tile_end = row_end - tile_r0 < tile_h ? row_end : tile_r0 + tile_h;
        for (int g = group_of_row(gt, tile_r0); g < gt.n && gt.off[g] < tile_end; ++g)
            if (gt.cnt[g] > 0) used |= 1u << (gt.off[g] <= tile_r0 ? 0 : (int)((gt.off[g] - tile_r0) / 16));
        for (uint32_t m = used; m != 0u; m &= m - 1u) {
            const int slot = __builtin_ctz(m);
            for (int i = threadIdx.x; i < kTileCols; i += 256) gred[slot][i] = 0u;
        }
        __syncthreads();
    }
    auto group_flush = [&](int g) {   // this wave's column maxima of expert g into its slot
        const int64_t o = gt.off[g];
        const int slot = o <= tile_r0 ? 0 : (int)((o - tile_r0) / 16);
        if (lane == 0) gslot[slot] = g;   // (the same g from every wave)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            atomicMax(&gred[slot][lane * 8 + 2 * k], cm[k] & 0xffffu);
            atomicMax(&gred[slot][lane * 8 + 2 * k + 1], cm[k] >> 16);
            cm[k] = 0u;
        }
    };
    // per-token and grouped: the row-pair maxima of each sub-block of each
    // wave, combined into row_amax after the loop (thread t: wave t / 64,
    // sub-block (t / 8) % 8, pair t % 8)
    constexpr bool kRows = KIND == AMAX_TOKEN || KIND == AMAX_GROUPED;
    __shared__ uint32_t rowred[kRows ? 4 : 1][kRows ? kAmaxRows / 64 : 1][8];
    auto flush_rows = [&]() {
        if (row_amax == nullptr) return;
        const int t = threadIdx.x, w = t >> 6, si = (t >> 3) & 7, jj = t & 7;
        const int64_t r0 = wave_row0(w) + si * rstride;
        if (16 * si < tile_h / 4 && r0 < row_end) {
            const uint32_t pair = rowred[w][si][jj];
            if (r0 + 2 * jj < row_end) atomic_max_mag(row_amax + r0 + 2 * jj, pair & 0xffffu);
            if (r0 + 2 * jj + 1 < row_end) atomic_max_mag(row_amax + r0 + 2 * jj + 1, pair >> 16);
        }
    };
    // The first 16-row sub-block is loaded here; each row of the next one is
    // loaded into the registers of the same row of the current one as soon as
    // that row's maxima are taken, so one set of data registers suffices.
    u32x4 v[16];
    if (rb < row_end) load_subblock(x, K, rb, row_end, lane_off, xr, v);
#pragma unroll 1
    for (int s = 0; s < tile_h / 4; s += 16) {
        const int64_t r0 = rb + (s >> 4) * rstride;
        if (r0 >= row_end) break;
        if (KIND == AMAX_GROUPED) {
            const int g = cur_group < 0 ? group_of_row(gt, r0) : group_advance(gt, cur_group, r0);
            if (g != cur_group) {
                if (cur_group >= 0) group_flush(cur_group);
                cur_group = g;
            }
        }
        // the next sub-block's rows (an empty buffer when there is none)
        const bool more = s + 16 < tile_h / 4 && r0 + rstride < row_end;
        const int64_t left = row_end - (r0 + rstride);
        const __amdgpu_buffer_rsrc_t nrs = more ? rsrc(x + (r0 + rstride) * K, (uint32_t)(left < 16 ? left : 16) * xr)
                                                : rsrc(x, 0u);
        uint32_t rm[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t a0 = abs2(v[i].x), a1 = abs2(v[i].y), a2 = abs2(v[i].z), a3 = abs2(v[i].w);
            rm[i] = max_halves(pk_max_u16(pk_max_u16(a0, a1), pk_max_u16(a2, a3)));
            cm[0] = pk_max_u16(cm[0], a0);
            cm[1] = pk_max_u16(cm[1], a1);
            cm[2] = pk_max_u16(cm[2], a2);
            cm[3] = pk_max_u16(cm[3], a3);
            uint32_t so = i * xr;
            asm volatile("" : "+s"(so) : "v"(rm[i]), "v"(cm[0]), "v"(cm[1]), "v"(cm[2]), "v"(cm[3]));
            v[i] = __builtin_amdgcn_raw_buffer_load_b128(nrs, lane_off, so, 0);
        }
        if (kRows && row_amax != nullptr) {
            uint32_t pair;
            const int j = wave_rowmax16(rm, &pair);
            if ((lane & 7) == 0) rowred[wave][s >> 4][j] = pair;
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
        if (threadIdx.x == 0 && zeroed()) {
            uint32_t m = tred[0];
            for (int w = 1; w < 4; ++w) m = m > tred[w] ? m : tred[w];
            if (t0) atomic_max_mag(t0, m);
            if (t1) atomic_max_mag(t1, m);
        }
        return;
    }
    if (KIND == AMAX_GROUPED) {
        if (cur_group >= 0) group_flush(cur_group);
        if (threadIdx.x == 0) zero_ok = zeroed();
        __syncthreads();
        if (!zero_ok) return;
        flush_rows();
        const int64_t tc0 = (int64_t)bx * kTileCols;
        for (uint32_t m = used; m != 0u; m &= m - 1u) {
            const int slot = __builtin_ctz(m);
            const int g = gslot[slot];
            for (int c = threadIdx.x; c < kTileCols; c += 256)
                if (tc0 + c < K) atomic_max_mag(col_amax + (int64_t)(gt.first + g) * K + tc0 + c, gred[slot][c]);
        }
        return;
    }
    // per token: the four waves' column maxima combined in LDS, then one
    // atomic per row and per column
    if (col_amax != nullptr) {
#pragma unroll
        for (int k = 0; k < 4; ++k) red[wave][lane][k] = cm[k];
    }
    if (threadIdx.x == 0) zero_ok = zeroed();
    __syncthreads();
    if (!zero_ok) return;
    flush_rows();
    if (col_amax != nullptr) {
        // thread t: the column pair 8 (t / 4) + 2 (t % 4) of the tile
        const int t = threadIdx.x, l = t >> 2, k = t & 3;
        const uint32_t m = pk_max_u16(pk_max_u16(red[0][l][k], red[1][l][k]), pk_max_u16(red[2][l][k], red[3][l][k]));
        const int64_t c = (int64_t)bx * kTileCols + 8 * l + 2 * k;
        if (c < K) {
            atomic_max_mag(col_amax + c, m & 0xffffu);
            atomic_max_mag(col_amax + c + 1, m >> 16);
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

// the same for a k known only at run time: the word is picked first and
// then shifted by an amount that depends on k, so that a loop over k does
// not get all eight unpacked values of every word hoisted out of it
__device__ __forceinline__ float elem_rt(const u32x4& w, int k) {
    const uint32_t word = (k >> 1) == 0 ? w.x : (k >> 1) == 1 ? w.y : (k >> 1) == 2 ? w.z : w.w;
    return __uint_as_float((word >> (16 * (k & 1))) << 16);
}

// Byte offset of scale (r, c) in the GEMM-swizzled layout of a scale matrix
// with nbp (a multiple of 4) blocks per row: 512-byte tiles of 128 rows x 4
// blocks, row-tile major; row r in 16-byte line r % 32 at 4-byte slot
// (r / 32) % 4, block c at byte c % 4.
__device__ __forceinline__ int64_t swz_offset(int64_t r, uint32_t c, uint32_t nbp) {
    return (r >> 7) * (128 * (int64_t)nbp) + (int64_t)(c >> 2) * 512 + (r & 31) * 16 + ((r >> 5) & 3) * 4 + (c & 3);
}

// Where a lane's sub-block results go.  Row and column bases are per
// sub-block; lane offsets are 32-bit.  Columnwise data of column c, rows
// [r0, r0+16) of a vector of length m_len starting at row grow0.
struct SubDst {
    uint8_t* row_q; uint8_t* row_sf;     // at row r0, column 0
    uint8_t* col_q; uint8_t* col_sf;     // at column 0 of this vector's slab, row r0
    uint32_t row_q_stride, row_sf_stride; // bytes per row: K/2, K/16
    uint32_t col_q_stride, col_sf_stride; // bytes per column: m_len/2, m_len/16
    uint32_t c0;                          // first column of this lane
    int nrows;                            // valid rows in the sub-block (<= 16)
    bool col_ok, odd;
    // columnwise output staged in LDS (when non-null): the lane's 8 columns
    // start at lds_q (pitch kStageQPitch bytes per column, this sub-block's
    // 8 bytes at the right offset) and lds_sf (pitch kStageSfPitch)
    uint8_t* lds_q; uint8_t* lds_sf;
};

// rowwise scale byte of row i of the sub-block, block c0 / 16.  SWZ: row_sf
// points at the swizzled position of (r0, block 0), r0 % 16 == 0, so rows
// r0 .. r0 + 15 share their 128-row group and 32-row slot.
template <bool SWZ>
__device__ __forceinline__ uint8_t* row_sf_at(const SubDst& d, int i) {
    const uint32_t c = d.c0 / 16;
    return SWZ ? d.row_sf + i * 16 + (c >> 2) * 512 + (c & 3) : d.row_sf + i * d.row_sf_stride + c;
}

template <bool SWZ>
__device__ __forceinline__ void store_row_pair(const SubDst& d, int i, uint32_t q0, uint32_t q1, uint32_t own_code) {
    if (!d.col_ok) return;
    if (i < d.nrows) __builtin_nontemporal_store(q0, reinterpret_cast<uint32_t*>(d.row_q + i * d.row_q_stride + d.c0 / 2));
    if (i + 1 < d.nrows) __builtin_nontemporal_store(q1, reinterpret_cast<uint32_t*>(d.row_q + (i + 1) * d.row_q_stride + d.c0 / 2));
    const int io = d.odd ? i + 1 : i;
    if (io < d.nrows) *row_sf_at<SWZ>(d, io) = (uint8_t)own_code;
}

template <bool SWZ>
__device__ __forceinline__ void store_row(const SubDst& d, int i, uint32_t q, uint32_t code) {
    if (d.col_ok && i < d.nrows) {
        *reinterpret_cast<uint32_t*>(d.row_q + i * d.row_q_stride + d.c0 / 2) = q;
        if (!d.odd) *row_sf_at<SWZ>(d, i) = (uint8_t)code;
    }
}

template <bool STAGE>
__device__ __forceinline__ void store_col(const SubDst& d, int j, uint32_t lo, uint32_t hi, uint32_t code) {
    if (!d.col_ok) return;
    if (STAGE) {
        *reinterpret_cast<u32x2*>(d.lds_q + j * kStageQPitch) = u32x2{lo, hi};
        d.lds_sf[j * kStageSfPitch] = (uint8_t)code;
        return;
    }
    const uint32_t c = d.c0 + j;
    *reinterpret_cast<u32x2*>(d.col_q + c * d.col_q_stride) = u32x2{lo, hi};
    d.col_sf[c * d.col_sf_stride] = (uint8_t)code;
}

// Exact encode and store of a sub-block with IEEE divisions throughout,
// re-reading the data from xr (row r0, column 0; row stride K).  rowA[i]:
// amax of row i; colA: this lane's 8 column amax; tileA: the tensor's.
template <bool ROW, bool COL, bool TILE, bool STAGE, bool SWZ>
__device__ __forceinline__ void encode_exact_body(const uint16_t* __restrict__ xr, int64_t K, const float* rowA,
                                                  const float* colA, float tileA, const SubDst& d) {
    u32x4 v[16];
    for (int i = 0; i < 16; ++i)
        v[i] = (d.col_ok && i < d.nrows) ? *reinterpret_cast<const u32x4*>(xr + i * K + d.c0) : u32x4{0u, 0u, 0u, 0u};
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
            if (ROW) store_row<SWZ>(d, i, w, bs.code);
        }
        if (COL)
            for (int j = 0; j < 8; ++j) {
                uint32_t lohi[2] = {0u, 0u};
                for (int i = 0; i < 16; i += 2)
                    lohi[i >> 3] |= (__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, quotient_exact(elem(v[i], j), bs),
                                                                         quotient_exact(elem(v[i + 1], j), bs), 1.0f, 0) & 0xffu) << (8 * ((i >> 1) & 3));
                store_col<STAGE>(d, j, lohi[0], lohi[1], bs.code);
            }
        return;
    }
    if (ROW) {
        for (int i = 0; i < 16; ++i) {
            uint32_t hw = rowmax_word(v[i]);
            hw = pk_max_u16(hw, from_pair(hw));
            const BlockScale bs = block_scale(max_halves(hw), outer_scale(rowA[i]));
            uint32_t w = 0u;
            for (int k = 0; k < 8; k += 2)
                w |= (__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, quotient_exact(elem(v[i], k), bs),
                                                              quotient_exact(elem(v[i], k + 1), bs), 1.0f, 0) & 0xffu) << (4 * k);
            store_row<SWZ>(d, i, w, bs.code);
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
            store_col<STAGE>(d, j, lohi[0], lohi[1], bs.code);
        }
    }
}

// the same, out of line (kept out of the hot loops' register allocation)
template <bool ROW, bool COL, bool TILE, bool STAGE, bool SWZ>
__device__ __noinline__ void encode_exact(const uint16_t* __restrict__ xr, int64_t K, const float* rowA,
                                          const float* colA, float tileA, SubDst d) {
    encode_exact_body<ROW, COL, TILE, STAGE, SWZ>(xr, K, rowA, colA, tileA, d);
}

// One workgroup (blockDim.x a multiple of 64, at most 1024): m = max(obs),
// then buf[0] = max(buf[0] * decay, m), in fp32.  red: 16 floats of LDS.
// Four independent 16-byte loads per thread per round keep the latency of a
// single pass over a few hundred KB low.
__device__ void wg_accumulate_reduce(float* __restrict__ buf, const float* __restrict__ obs, int64_t n, float decay,
                                     float* red) {
    float m = 0.0f;
    const int64_t nv = (reinterpret_cast<uintptr_t>(obs) % 16 == 0) ? n / 4 : 0;   // float4 part
    const float4* o4 = reinterpret_cast<const float4*>(obs);
    for (int64_t i = threadIdx.x; i < nv; i += 4 * blockDim.x) {
        float4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t j = i + k * (int64_t)blockDim.x;
            v[k] = j < nv ? o4[j] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            m = v[k].x > m ? v[k].x : m; m = v[k].y > m ? v[k].y : m;
            m = v[k].z > m ? v[k].z : m; m = v[k].w > m ? v[k].w : m;
        }
    }
    for (int64_t i = 4 * nv + threadIdx.x; i < n; i += blockDim.x) m = obs[i] > m ? obs[i] : m;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const float o = __shfl_xor(m, d);
        m = o > m ? o : m;
    }
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        const int nw = (int)(blockDim.x >> 6);
        for (int w = 1; w < nw; ++w) m = red[w] > m ? red[w] : m;
        const float t = buf[0] * decay;
        buf[0] = m > t ? m : t;
    }
}

// MODE: ENC_TENSOR (row_amax[0] / col_amax[0] for every vector), ENC_TOKEN
// (row_amax[r], col_amax[c]), ENC_TILE (16x16 tiles, tensor amax in
// row_amax[0] or col_amax[0]; also fills row_amax[1..M) and col_amax[1..K)
// with it), ENC_GROUPED (rowwise per-token; columnwise per expert with
// col_amax[e][K] and per-expert output slabs).  A workgroup covers kEncRows
// (256) rows x 256 columns: each wave takes a quarter of the rows in steps of
// 32, a step being two groups of 32 lanes with a 16-row x 8-column sub-block
// per lane.  SAT:
// the amax comes from the caller and may be smaller than the data.
// Requires K < 2^25 (32 rows of a step span less than 2^31 bytes).
//
// A step: (1) sixteen 16-byte loads; (2) column maxima and the rowwise block
// maxima from the packed words, then the block parameters of the lane's 8
// column blocks; (3) per row pair, the rowwise block parameters of the
// lane's own row (2s + parity, swapped with the pair through DPP), the two
// rows unpacked once and encoded both ways.  Rowwise bytes go straight to
// memory; columnwise bytes are staged in LDS and written in whole lines at
// the end of the workgroup's tile.
// SWZ (per-tensor and per-token casts of M % 128 == 0, K % 128 == 0 only):
// both scale outputs in the GEMM-swizzled layout (swz_offset; the rowwise
// matrix is [M][K/16], the columnwise [K][M/16]), each workgroup writing whole
// 512-byte tiles of it.
template <int MODE, bool ROW, bool COL, bool SAT, bool SWZ>
__global__ __launch_bounds__(256) void k_encode(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                int64_t row_begin, int64_t row_end,
                                                const float* __restrict__ row_amax, const float* __restrict__ col_amax,
                                                uint8_t* __restrict__ row_q, uint8_t* __restrict__ row_sf,
                                                uint8_t* __restrict__ col_q, uint8_t* __restrict__ col_sf,
                                                float* __restrict__ fill_row, float* __restrict__ fill_col,
                                                GroupTable gt, Calib cal, int tile_h) {
    constexpr bool TILE = MODE == ENC_TILE;
    constexpr bool ROWTOK = ROW && !TILE && MODE != ENC_TENSOR;   // a row amax per row
    __shared__ float row_scale[4][32][2];    // per wave: S and 1/S of the step's 32 rows
    // columnwise output of the workgroup tile, written out in whole lines
    constexpr bool STAGE = COL;
    __shared__ __attribute__((aligned(16))) uint8_t stage_q[STAGE ? kEncCols * kStageQPitch : 16];
    __shared__ __attribute__((aligned(16))) uint8_t stage_sf[STAGE ? kEncCols * kStageSfPitch : 16];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Workgroups are dispatched round-robin over the 8 XCDs (each with its
    // own L2).  Give XCD x a contiguous run of tiles, row band major, so the
    // scale bytes that share a cache line (rowwise: 4 adjacent column tiles,
    // columnwise: 8 adjacent row bands) are written through one L2.  The
    // tiles are walked in the amax pass's order (each XCD down its run of row
    // bands, as the amax pass read them): in the steady state this measured
    // faster than the reverse walk.
    const uint32_t ntiles = gridDim.x * gridDim.y;
    const uint32_t lin = blockIdx.y * gridDim.x + blockIdx.x;
    uint32_t tile = lin;
    if ((ntiles & 7u) == 0u) tile = (lin & 7u) * (ntiles >> 3) + (lin >> 3);
    const uint32_t bx = tile % gridDim.x, by = tile / gridDim.x;
    const int rg = lane >> 5;                     // row group within the wave
    const uint32_t c0 = bx * kEncCols + (lane & 31) * 8;
    const bool col_ok = c0 < K;
    const bool odd = lane & 1;
    const int64_t tile_r0 = row_begin + (int64_t)by * tile_h;   // tile_h: 128 or 256 rows
    const int64_t wbase = tile_r0 + wave * (tile_h / 4);   // a wave covers tile_h/4 rows in 32-row steps
    float tileA = 0.0f;
    if (TILE) {
        tileA = row_amax ? row_amax[0] : col_amax[0];
        const int64_t gid = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
        const int64_t gsz = (int64_t)gridDim.x * gridDim.y * blockDim.x;
        if (fill_row) for (int64_t i = 1 + gid; i < M; i += gsz) fill_row[i] = tileA;
        if (fill_col) for (int64_t i = 1 + gid; i < K; i += gsz) fill_col[i] = tileA;
    }
    const Outer tileO = make_outer(tileA);
    // the calibration update, folded into the cast: one workgroup reduces the
    // finished amax vector into the decayed buffer
    if (cal.buf != nullptr && lin == 0u) {
        wg_accumulate_reduce(cal.buf, cal.obs, cal.n, cal.decay, &row_scale[0][0][0]);
        __syncthreads();
    }

    // columnwise outer scales of this lane's 8 columns: per-token casts keep
    // the tile's 256 in LDS (every lane of a column reads the same entry),
    // the others in registers
    constexpr bool COL_LDS = COL && MODE == ENC_TOKEN;
    __shared__ float2 col_scale[COL_LDS ? kEncCols : 1];
    Outer colO[8];
    bool col_slow = false;
    int cur_group = -1;    // the lane's expert (grouped casts)
    int wave_group = -1;   // expert of the wave's current first row
    int64_t m_len = M, grow0 = 0;
    if (COL_LDS) {
        // one column per thread; a column outside the fast range sends the
        // whole tile to the exact path
        const uint32_t c = bx * kEncCols + threadIdx.x;
        const Outer o = make_outer<SAT>(c < K ? col_amax[c] : 0.0f, c < K);
        col_scale[threadIdx.x] = make_float2(o.S, o.yS);
        col_slow = __syncthreads_or(o.slow) != 0;
    } else if (COL && !TILE && MODE != ENC_GROUPED) {
        const float ca = col_amax[0];
#pragma unroll
        for (int j = 0; j < 8; ++j) colO[j] = make_outer<SAT>(ca);
        col_slow = colO[0].slow;
    }
    // per-tensor rowwise outer scale
    const float rowA_t = (ROW && MODE == ENC_TENSOR) ? row_amax[0] : 0.0f;
    const Outer rowO_t = make_outer<SAT>(rowA_t, ROW && MODE == ENC_TENSOR);
    const bool tile_slow = (TILE && tileO.slow) || (ROW && MODE == ENC_TENSOR && rowO_t.slow);

    // destinations of a sub-block (columnwise output and the exact path)
    auto make_dst = [&](int64_t r0, int nrows, int64_t mlen, int64_t g0) {
        SubDst d;
        d.row_q = row_q + r0 * (K / 2);
        d.row_sf = SWZ ? row_sf + swz_offset(r0, 0u, (uint32_t)(K / 16)) : row_sf + r0 * (K / 16);
        d.col_q = col_q + g0 * K / 2 + (r0 - g0) / 2;
        d.col_sf = col_sf + g0 * K / 16 + (r0 - g0) / 16;
        d.row_q_stride = (uint32_t)(K / 2);
        d.row_sf_stride = (uint32_t)(K / 16);
        d.col_q_stride = (uint32_t)(mlen / 2);
        d.col_sf_stride = (uint32_t)(mlen / 16);
        d.c0 = c0; d.nrows = nrows; d.col_ok = col_ok; d.odd = odd;
        d.lds_q = nullptr; d.lds_sf = nullptr;
        if (STAGE) {
            const int rl = (int)(r0 - tile_r0);   // row within the tile
            d.lds_q = stage_q + ((lane & 31) * 8) * kStageQPitch + rl / 2;
            d.lds_sf = stage_sf + ((lane & 31) * 8) * kStageSfPitch + rl / 16;
        }
        return d;
    };

    // lane parts of the buffer offsets within a step (row group, column)
    const uint32_t xrow = (uint32_t)K * 2u, qrow = (uint32_t)(K / 2), srow = (uint32_t)(K / 16);
    const uint32_t vx = col_ok ? 16u * rg * xrow + c0 * 2u : kOffOut;
    const uint32_t vq = col_ok ? 16u * rg * qrow + c0 / 2u : kOffOut;
    // swizzled rowwise scales: the lane's row line and block byte within the
    // step's 128-row group (the step's 32-row slot goes in the scalar offset)
    const uint32_t vs = !col_ok ? kOffOut
                        : SWZ ? ((c0 / 16u) >> 2) * 512u + ((c0 / 16u) & 3u) + (16u * rg + (odd ? 1u : 0u)) * 16u
                              : (16u * rg + (odd ? 1u : 0u)) * srow + c0 / 16u;
    // v_perm selector moving this lane's row (low half: even, high: odd) to the top half
    const uint32_t own_sel = odd ? 0x03020c0cu : 0x01000c0cu;

    uint32_t slow_mask = 0u;
    constexpr int kSteps = kEncRows / 4 / 32;   // 32-row steps per wave
    // loads of a step issued during the step before it (grouped casts, which
    // keep their expert's column scales in registers, load at the step's top)
    constexpr bool kPrefetch = MODE != ENC_GROUPED;
    // Valid rows of step sb (0 for a wave whose rows all lie past the end:
    // its first step's loads are issued before the step loop's exit test).
    auto step_rows = [&](int sb) -> uint32_t {
        const int64_t left = row_end - (wbase + 32 * sb);
        return left <= 0 ? 0u : (left < 32 ? (uint32_t)left : 32u);
    };
    // The x buffer of a step spans its valid rows only, so that rows past the
    // end read zeros without a memory access (and their stores below are
    // dropped); an empty step gets an empty buffer.
    auto x_rsrc = [&](int sb) {
        return rsrc(x + (wbase + 32 * sb) * K, step_rows(sb) * xrow);
    };
    auto load_ra = [&](int sb) -> float {
        if (!ROWTOK) return 0.0f;
        const uint32_t l = (uint32_t)(lane & 31);
        return row_amax[l < step_rows(sb) ? wbase + 32 * sb + l : row_begin];
    };
    // The row stride is made opaque: otherwise the compiler keeps the 16
    // per-row lane offsets live in registers instead of putting each row's in
    // the scalar offset where it is used.
    uint32_t xr = xrow;
    asm volatile("" : "+s"(xr));
    // The first step's rows are loaded here; each later step's rows are loaded
    // during the step before it, a row pair at a time, into the registers of
    // the pair just encoded, so a wave waits for memory once per tile and
    // needs no second set of data registers.
    u32x4 v[16];
    float ra = load_ra(0);
    {
        const __amdgpu_buffer_rsrc_t rs = x_rsrc(0);
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, vx, i * xr, kCacheNT);
    }
#pragma unroll
    for (int sb = 0; sb < kSteps; ++sb) {
        const int64_t wr0 = wbase + 32 * sb;     // first row of the wave's step
        if (32 * sb >= tile_h / 4 || wr0 >= row_end) break;
        const uint32_t nrows = (uint32_t)(row_end - wr0 < 32 ? row_end - wr0 : 32);   // rows of the step
        const bool group_ok = 16u * rg < nrows;
        const int64_t r0 = group_ok ? wr0 + 16 * rg : wr0;
        // the next step's rows (an empty buffer when there is none: its loads
        // then return zeros without touching memory)
        const bool more = sb + 1 < kSteps && 32 * (sb + 1) < tile_h / 4 && wr0 + 32 < row_end;
        if (sb > 0 && !kPrefetch) {
            const __amdgpu_buffer_rsrc_t rs = x_rsrc(sb);
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, vx, i * xr, kCacheNT);
            ra = load_ra(sb);
        }
        const __amdgpu_buffer_rsrc_t nx_rs = more ? x_rsrc(sb + 1) : rsrc(x, 0u);
        // rows i, i+1 of the next step, loaded once the outputs of the pair
        // that held them (d0, d1: its rowwise words; dc: its columnwise
        // words) are computed, so that they land in that pair's registers
        auto load_next = [&](int i, uint32_t d0, uint32_t d1, const uint32_t* dc) {
            uint32_t so = i * xr;
            asm volatile("" : "+s"(so) : "v"(d0), "v"(d1), "v"(dc[0]), "v"(dc[2]), "v"(dc[4]), "v"(dc[6]),
                         "v"(dc[8]), "v"(dc[10]), "v"(dc[12]), "v"(dc[14]));
            v[i] = __builtin_amdgcn_raw_buffer_load_b128(nx_rs, vx, so, kCacheNT);
            v[i + 1] = __builtin_amdgcn_raw_buffer_load_b128(nx_rs, vx, so + xr, kCacheNT);
        };
        uint32_t qr = qrow, sr = srow;
        asm volatile("" : "+s"(qr), "+s"(sr));
        if (COL && MODE == ENC_GROUPED) {
            // the experts of the step's two row groups, found wave-uniformly
            // (scalar loads of the table) from the wave's cursor, then each
            // lane takes its group's
            wave_group = wave_group < 0 ? group_of_row(gt, wr0) : group_advance(gt, wave_group, wr0);
            const int g0 = wave_group;
            const int g1 = nrows > 16u ? group_advance(gt, g0, wr0 + 16) : g0;
            const int g = rg ? g1 : g0;
            if (g != cur_group) {
                cur_group = g;
                m_len = gt.cnt[g];
                grow0 = gt.off[g];
                const int64_t base = (int64_t)(gt.first + g) * K;
                float ca[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) ca[j] = col_amax[base + (col_ok ? c0 + j : 0)];
                col_slow = false;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    colO[j] = make_outer(col_ok ? ca[j] : 0.0f);
                    col_slow |= colO[j].slow;
                }
            }
        }
        SubDst d = make_dst(r0, group_ok ? (int)(nrows - 16u * rg < 16u ? nrows - 16u * rg : 16u) : 1, m_len, grow0);
        if (!group_ok) { d.nrows = 0; d.col_ok = false; }

        // rowwise outer scales: lanes 0..31 compute one row of the step each
        // into LDS; a row outside the fast range sends the whole step to the
        // exact path
        bool step_slow = tile_slow;
        if (ROWTOK) {
            const bool row_in = (uint32_t)(lane & 31) < nrows;
            const Outer o = make_outer<SAT>(row_in ? ra : 0.0f, row_in);
            if (kPrefetch && more) ra = load_ra(sb + 1);
            if (lane < 32) {
                row_scale[wave][lane][0] = o.S;
                row_scale[wave][lane][1] = o.yS;
            }
            step_slow |= __builtin_amdgcn_ballot_w64(o.slow) != 0ull;
            // other lanes read these entries below: the fence keeps the
            // compiler from moving those reads above the writes (a wave
            // executes its LDS instructions in order)
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }

        // (2) maxima from the packed words
        bool slow = col_slow;
        uint32_t cm[4] = {0u, 0u, 0u, 0u};    // columns 2k (low half) and 2k+1 (high half)
        uint32_t bm[8];                       // rowwise block max of the own row of pair s
        uint32_t tm = 0u;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            uint32_t rw[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32x4 w = v[2 * s + h];
                const uint32_t a0 = abs2(w.x), a1 = abs2(w.y), a2 = abs2(w.z), a3 = abs2(w.w);
                if (COL && !TILE) {
                    cm[0] = pk_max_u16(cm[0], a0);
                    cm[1] = pk_max_u16(cm[1], a1);
                    cm[2] = pk_max_u16(cm[2], a2);
                    cm[3] = pk_max_u16(cm[3], a3);
                }
                rw[h] = pk_max_u16(pk_max_u16(a0, a1), pk_max_u16(a2, a3));
            }
            if (TILE) {
                tm = pk_max_u16(tm, pk_max_u16(rw[0], rw[1]));
            } else if (ROW) {
                // (row 2s | row 2s+1 << 16) over the lane's 8 columns, then the pair's 16
                uint32_t m = pk_max_u16(__builtin_amdgcn_perm(rw[1], rw[0], 0x05040100u),
                                        __builtin_amdgcn_perm(rw[1], rw[0], 0x07060302u));
                m = pk_max_u16(m, from_pair(m));
                bm[s] = __builtin_amdgcn_perm(m, m, own_sel);
            }
        }
        // the rowwise block maxima are finished here, so that the 64 absolute
        // values they come from are dead before the row pairs start (left to
        // itself the compiler computes each pair's maximum where it is used)
        if (ROW && !TILE)
            asm volatile("" : "+v"(bm[0]), "+v"(bm[1]), "+v"(bm[2]), "+v"(bm[3]),
                         "+v"(bm[4]), "+v"(bm[5]), "+v"(bm[6]), "+v"(bm[7]));
        // block parameters of the lane's column blocks (or of its 16x16 tile)
        FastBlock cb[8];
        FastBlock tb;
        if (TILE) {
            const uint32_t m = pk_max_u16(tm, from_pair(tm));
            tb = fast_block<SAT>(max_halves(m) << 16, tileO);
            slow |= tb.slow;
        } else if (COL) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t bits = (j & 1) ? (cm[j >> 1] & 0xffff0000u) : (cm[j >> 1] << 16);
                Outer o = colO[j];
                if (COL_LDS) {
                    const float2 sy = col_scale[(lane & 31) * 8 + j];
                    o.S = sy.x;
                    o.yS = sy.y;
                }
                cb[j] = fast_block<SAT, !SAT>(bits, o);
                slow |= cb[j].slow;
                // the scale byte goes to the staging area now rather than
                // being held through the row pairs
                if (d.col_ok) d.lds_sf[j * kStageSfPitch] = (uint8_t)cb[j].code;
            }
        }

        // (3) per row pair: rowwise parameters, then both encodings
        const __amdgpu_buffer_rsrc_t q_rs = rsrc(row_q + wr0 * (K / 2), nrows * qrow);
        // (swizzled: every step is 32 whole rows, M % 128 == 0)
        const __amdgpu_buffer_rsrc_t s_rs = SWZ ? rsrc(row_sf + (wr0 >> 7) * 128 * (K / 16), 128u * srow)
                                                : rsrc(row_sf + wr0 * (K / 16), nrows * srow);
        const uint32_t s_slot = SWZ ? (uint32_t)((wr0 >> 5) & 3) * 4u : 0u;
        uint32_t cq[8][2] = {};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int i = 2 * s;
            float yh0 = 0.0f, yl0 = 0.0f, yh1 = 0.0f, yl1 = 0.0f;
            if (ROW) {
                if (TILE) {
                    yh0 = yh1 = tb.yh;
                    yl0 = yl1 = tb.yl;
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)tb.code, s_rs, vs, i * sr, 0);
                } else {
                    Outer ro = rowO_t;
                    if (ROWTOK) {
                        ro.S = row_scale[wave][16 * rg + i + (odd ? 1 : 0)][0];
                        ro.yS = row_scale[wave][16 * rg + i + (odd ? 1 : 0)][1];
                    }
                    const FastBlock f = fast_block<SAT, !SAT>(bm[s], ro);
                    slow |= f.slow;
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)f.code, s_rs, vs, SWZ ? i * 16u + s_slot : i * sr, 0);
                    yh0 = from_even(f.yh); yl0 = from_even(f.yl);
                    yh1 = from_odd(f.yh);  yl1 = from_odd(f.yl);
                }
            }
            // The empty asm orders the row pairs: pair s is unpacked (16
            // registers) only after pair s-1's stores and columnwise nibbles
            // are done.  Otherwise the rowwise halves of all pairs run as
            // soon as their rows arrive and every unpacked value stays live
            // until the columnwise block parameters are known.
            u32x4 w0 = v[i], w1 = v[i + 1];
            if (COL && s > 0)
                asm volatile("" : "+v"(w0), "+v"(w1), "+v"(cq[0][(s - 1) >> 2]), "+v"(cq[1][(s - 1) >> 2]),
                             "+v"(cq[2][(s - 1) >> 2]), "+v"(cq[3][(s - 1) >> 2]), "+v"(cq[4][(s - 1) >> 2]),
                             "+v"(cq[5][(s - 1) >> 2]), "+v"(cq[6][(s - 1) >> 2]), "+v"(cq[7][(s - 1) >> 2]));
            else
                asm volatile("" : "+v"(w0), "+v"(w1));
            const float a0[8] = {bf_lo(w0.x), bf_hi(w0.x), bf_lo(w0.y), bf_hi(w0.y),
                                 bf_lo(w0.z), bf_hi(w0.z), bf_lo(w0.w), bf_hi(w0.w)};
            const float a1[8] = {bf_lo(w1.x), bf_hi(w1.x), bf_lo(w1.y), bf_hi(w1.y),
                                 bf_lo(w1.z), bf_hi(w1.z), bf_lo(w1.w), bf_hi(w1.w)};
            if (COL) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float yh = TILE ? tb.yh : cb[j].yh, yl = TILE ? tb.yl : cb[j].yl;
                    const float q0 = quot2(a0[j], yh, yl), q1 = quot2(a1[j], yh, yl);
                    uint32_t& w = cq[j][s >> 2];
                    // byte 0 first: the bytes above it are written by the next
                    // three conversions, so the register merged into can be q0's
                    if ((s & 3) == 0) w = put_fp4x2<0>(__float_as_uint(q0), q0, q1);
                    else if ((s & 3) == 1) w = put_fp4x2<1>(w, q0, q1);
                    else if ((s & 3) == 2) w = put_fp4x2<2>(w, q0, q1);
                    else w = put_fp4x2<3>(w, q0, q1);
                }
            }
            uint32_t o0 = 0u, o1 = 0u;
            if (ROW) {
                // as above: bytes 1..3 overwrite whatever byte 0's conversion kept
                const float p00 = quot2(a0[0], yh0, yl0), p10 = quot2(a1[0], yh1, yl1);
                o0 = put_fp4x2<0>(__float_as_uint(p00), p00, quot2(a0[1], yh0, yl0));
                o0 = put_fp4x2<1>(o0, quot2(a0[2], yh0, yl0), quot2(a0[3], yh0, yl0));
                o0 = put_fp4x2<2>(o0, quot2(a0[4], yh0, yl0), quot2(a0[5], yh0, yl0));
                o0 = put_fp4x2<3>(o0, quot2(a0[6], yh0, yl0), quot2(a0[7], yh0, yl0));
                o1 = put_fp4x2<0>(__float_as_uint(p10), p10, quot2(a1[1], yh1, yl1));
                o1 = put_fp4x2<1>(o1, quot2(a1[2], yh1, yl1), quot2(a1[3], yh1, yl1));
                o1 = put_fp4x2<2>(o1, quot2(a1[4], yh1, yl1), quot2(a1[5], yh1, yl1));
                o1 = put_fp4x2<3>(o1, quot2(a1[6], yh1, yl1), quot2(a1[7], yh1, yl1));
                __builtin_amdgcn_raw_buffer_store_b32(o0, q_rs, vq, i * qr, kCacheNT);
                __builtin_amdgcn_raw_buffer_store_b32(o1, q_rs, vq, (i + 1) * qr, kCacheNT);
            }
            if (kPrefetch && sb + 1 < kSteps) load_next(i, o0, o1, &cq[0][s >> 2]);
        }
        if (COL) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (TILE) store_col<STAGE>(d, j, cq[j][0], cq[j][1], tb.code);
                else if (d.col_ok) *reinterpret_cast<u32x2*>(d.lds_q + j * kStageQPitch) = u32x2{cq[j][0], cq[j][1]};
            }
        }
        if (step_slow || __builtin_amdgcn_ballot_w64(slow) != 0ull) slow_mask |= 1u << sb;
        // the next step's row scales overwrite entries other lanes read above
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }

    // sub-blocks with a block outside the fast path's range: encode again,
    // exactly, over what the fast path stored
    while (slow_mask != 0u) {
        const int sb = __builtin_ctz(slow_mask);
        slow_mask &= slow_mask - 1u;
        const int64_t wr0 = wbase + 32 * sb;
        const bool group_ok = wr0 + 16 * rg < row_end;
        const int64_t r0 = group_ok ? wr0 + 16 * rg : wr0;
        const int nrows = group_ok ? (int)(row_end - r0 < 16 ? row_end - r0 : 16) : 1;
        int64_t mlen = M, g0 = 0, cbase = 0;
        if (COL && MODE == ENC_GROUPED) {
            const int g = group_of_row(gt, r0);
            mlen = gt.cnt[g];
            g0 = gt.off[g];
            cbase = (int64_t)(gt.first + g) * K;
        }
        float rowA[16], colA[8];
        for (int i = 0; i < 16; ++i)
            rowA[i] = (ROW && !TILE) ? (MODE == ENC_TENSOR ? rowA_t : (i < nrows ? row_amax[r0 + i] : 0.0f)) : 0.0f;
        for (int j = 0; j < 8; ++j)
            colA[j] = (COL && !TILE) ? (MODE == ENC_TENSOR ? col_amax[0] : (col_ok ? col_amax[cbase + c0 + j] : 0.0f)) : 0.0f;
        SubDst d = make_dst(r0, nrows, mlen, g0);
        if (!group_ok) { d.nrows = 0; d.col_ok = false; }
        encode_exact<ROW, COL, TILE, STAGE, SWZ>(x + r0 * K, K, rowA, colA, tileA, d);
    }

    if (STAGE) {
        // Every wave's columnwise bytes are in LDS: write them out in 16-byte
        // pieces along each column (whole 128-byte lines for a full tile),
        // then the scale bytes.  A grouped cast writes each expert's rows of
        // the tile into that expert's slab, one segment per expert.
        __syncthreads();
        const int64_t tile_rows = row_end - tile_r0 < tile_h ? row_end - tile_r0 : tile_h;
        const int64_t tile_end = tile_r0 + tile_rows;
        const uint32_t cbase = bx * kEncCols;
        const uint32_t ncols = (uint32_t)(K - cbase < kEncCols ? K - cbase : kEncCols);
        const uint32_t t = threadIdx.x;
        int e = MODE == ENC_GROUPED ? group_of_row(gt, tile_r0) : 0;
        for (int64_t s0 = tile_r0; s0 < tile_end;) {
            int64_t o = 0, m = M;   // first row and length of the vectors (the expert's for grouped)
            if (MODE == ENC_GROUPED) {
                while (gt.cnt[e] == 0 || gt.off[e] + gt.cnt[e] <= s0) ++e;
                o = gt.off[e];
                m = gt.cnt[e];
            }
            const int64_t s1 = o + m < tile_end ? o + m : tile_end;
            const uint32_t lq = (uint32_t)(s0 - tile_r0) / 2, qb = (uint32_t)(s1 - s0) / 2;    // multiples of 8
            const uint32_t ls = (uint32_t)(s0 - tile_r0) / 16, sbn = (uint32_t)(s1 - s0) / 16;
            uint8_t* gq = col_q + o * K / 2 + (s0 - o) / 2 + (int64_t)cbase * (m / 2);
            uint8_t* gs = col_sf + o * K / 16 + (s0 - o) / 16 + (int64_t)cbase * (m / 16);
            const int64_t qstride = m / 2, sstride = m / 16;
            // data: a segment is at most kEncRows/2 bytes per column, kNP
            // 16-byte pieces; thread t writes piece t % kNP (the segment's
            // last may be 8 bytes) of columns t / kNP, t / kNP + 256 / kNP, ...
            constexpr uint32_t kNP = kEncRows / 32;
            const uint32_t chunk = (t % kNP) * 16u;
            if (chunk < qb) {
                const bool whole = chunk + 16u <= qb;
                const uint8_t* src = stage_q + (t / kNP) * kStageQPitch + lq + chunk;
                uint8_t* dst = gq + (int64_t)(t / kNP) * qstride + chunk;
                for (uint32_t c = t / kNP; c < ncols; c += 256 / kNP) {
                    const u32x2 lo = *reinterpret_cast<const u32x2*>(src);
                    if (whole) {
                        const u32x2 hi = *reinterpret_cast<const u32x2*>(src + 8);
                        __builtin_nontemporal_store(u32x4{lo.x, lo.y, hi.x, hi.y}, reinterpret_cast<u32x4*>(dst));
                    } else {
                        __builtin_nontemporal_store(lo, reinterpret_cast<u32x2*>(dst));
                    }
                    src += (256 / kNP) * kStageQPitch;
                    dst += (256 / kNP) * qstride;
                }
            }
            // scale bytes: 16-byte pieces along each column (thread t: column
            // t) when the segment is a multiple of 256 rows and the destination
            // is aligned for them, else words, else bytes.  Swizzled: column
            // t's four blocks of each 4-block group as one word into the
            // group's 512-byte tile (the workgroup writes whole tiles).
            if (SWZ) {
                if (t < ncols) {
                    const uint32_t nbpc = (uint32_t)(M / 16);
                    const int64_t k = (int64_t)cbase + t;
                    for (uint32_t part = 0; part < sbn; part += 4) {
                        const uint32_t w = *reinterpret_cast<const uint32_t*>(stage_sf + t * kStageSfPitch + ls + part);
                        *reinterpret_cast<uint32_t*>(col_sf + swz_offset(k, (uint32_t)(s0 / 16) + part, nbpc)) = w;
                    }
                }
            } else if (sbn % 16 == 0 && ls % 4 == 0 && sstride % 16 == 0 && reinterpret_cast<uintptr_t>(gs) % 16 == 0) {
                if (t < ncols) {
                    for (uint32_t part = 0; part < sbn; part += 16) {
                        const uint32_t* src = reinterpret_cast<const uint32_t*>(stage_sf + t * kStageSfPitch + ls + part);
                        __builtin_nontemporal_store(u32x4{src[0], src[1], src[2], src[3]},
                                                    reinterpret_cast<u32x4*>(gs + (int64_t)t * sstride + part));
                    }
                }
            } else {
                const bool words = sbn % 4 == 0 && ls % 4 == 0 && sstride % 4 == 0 && reinterpret_cast<uintptr_t>(gs) % 4 == 0;
                for (uint32_t c = t; c < ncols; c += 256) {
                    const uint8_t* src = stage_sf + c * kStageSfPitch + ls;
                    uint8_t* dst = gs + (int64_t)c * sstride;
                    if (words) {
                        for (uint32_t b = 0; b < sbn; b += 4)
                            *reinterpret_cast<uint32_t*>(dst + b) = *reinterpret_cast<const uint32_t*>(src + b);
                    } else {
                        for (uint32_t b = 0; b < sbn; ++b) dst[b] = src[b];
                    }
                }
            }
            s0 = s1;
            if (MODE == ENC_GROUPED) ++e;
        }
    }
}

// ------------------------------------------------- stochastic rounding

// Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and
// Shaw ("Parallel random numbers: as easy as 1, 2, 3", SC'11): ten rounds of
// the two-multiplier S-box on the counter words, the key advanced by the
// two Weyl constants between rounds.
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        // one 32 x 32 -> 64-bit product per multiplier (v_mad_u64_u32), not
        // separate high and low multiplies
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t h0 = (uint32_t)(p0 >> 32), l0 = (uint32_t)p0;
        const uint32_t h1 = (uint32_t)(p1 >> 32), l1 = (uint32_t)p1;
        // each three-way xor as one v_bitop3_b32 (truth table 0x96)
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32(h1, c1, k0, 0x96), n2 = __builtin_amdgcn_bitop3_b32(h0, c3, k1, 0x96);
        c0 = n0;
        c1 = l1;
        c2 = n2;
        c3 = l0;
    }
    return u32x4{c0, c1, c2, c3};
}

// Stochastic E2M1 nibble of q with the 8-bit random byte K of word w: x = |q|
// lies in [lo, lo + d) of the E2M1 grid (d = 0.5 below 2, 1 below 4, 2
// below 6) and rounds up iff x - lo > U * d with U = R * 2^-8, R that byte;
// x >= 6 saturates; the sign bit of q is copied.  Without branches, through
// t = code(lo) * 2^22 + (x - lo) / d * 2^22 rounded up to an integer: at or
// above 1 that is exactly x's bit pattern less 252 * 2^22 (the exponent and
// first mantissa bit give the code, the other 22 bits (x - lo) / d); below 1
// it is ceil(x * 2^23) (lo = 0 or 0.5, d = 0.5).  Rounding up to the integer
// keeps the strict comparison exact, as R * 2^14 is an integer: x - lo >
// U * d iff t's low 22 bits exceed R * 2^14, compared here as t << 10 >
// R << 24; a carry into the code bits is a round-up, which the rule also
// takes there.  (tests/native/sr_round_check.c compares this form with the
// oracle's rule over every fp32 q.)
template <int K>
__device__ __forceinline__ uint32_t e2m1_sr(float q, uint32_t w) {
    const uint32_t b = __float_as_uint(q);
    const uint32_t xb = b & 0x7fffffffu;
    const uint32_t ta = xb - 0x3f000000u;
    const uint32_t tb = (uint32_t)__builtin_ceilf(__uint_as_float(xb < 0x3f800000u ? xb : 0x3f800000u) * 0x1p23f);
    const uint32_t t = xb >= 0x3f800000u ? ta : tb;
    const uint32_t r24 = __builtin_amdgcn_perm(0u, w, ((uint32_t)K << 24) | 0x000c0c0cu);   // byte K, shifted to the top
    const uint32_t c = (t >> 22) + ((t << 10) > r24 ? 1u : 0u);
    return ((b >> 28) & 8u) | (c < 7u ? c : 7u);
}

// the nibble of element k (0..7) of a lane's row from the row's two random
// words (bytes 0..3 of w0, then of w1)
template <int k>
__device__ __forceinline__ uint32_t e2m1_sr8(float q, uint32_t w0, uint32_t w1) {
    return e2m1_sr<k & 3>(q, k < 4 ? w0 : w1);
}

// Block parameters of the stochastic-rounding cast on the fast path: the
// exact block scale (code = E4M3(RN(RN(b / 6) / S)), r = decode(code) * S)
// from the division shortcut of fact 1 and 1b, and y = RN(1/r) for the
// element quotients RN(a / r) (fact 1).  slow: the vector's outer scale is
// outside the fast range, the scale falls in the E4M3 subnormal range, or r
// lies outside [2^-64, 2^64]; that block takes IEEE divisions throughout.
// An all-zero block gets code 0 and some normal r: its quotients are +/-0.
struct SrBlock {
    float r, y;
    uint32_t code;
    bool slow;
};

__device__ __forceinline__ SrBlock sr_block(uint32_t bbits, const Outer& o) {
    SrBlock f;
    const float t = div_fast(__uint_as_float(bbits), 6.0f, kRcp6);   // RN(b / 6)
    const float sf = div_fast(t, o.S, o.yS);                         // RN(t / S)
    const uint32_t u = __float_as_uint(sf);
    // E4M3 code by rounding sf's encoding (as in fast_block): the low byte
    uint32_t c = (u + (0x7FFFFu + (0x40u << 20)) + ((u >> 20) & 1u)) >> 20;
    c = c < 0x400u ? 0x400u : (c > 0x47Eu ? 0x47Eu : c);
    f.code = c & 0xffu;
    f.r = __uint_as_float((c << 20) - (0x40u << 20)) * o.S;
    f.y = rcp_rn(f.r);
    f.slow = o.slow || (u - 1u) < (0x3C800000u - 1u) || !(f.r >= 0x1p-64f && f.r <= 0x1p64f);
    return f;
}

// Stochastic-rounding cast (per-tensor or per-token outer amax, computed
// beforehand).  Block scales and element quotients are the exact IEEE ones of
// the deterministic cast; element i of a vector (a row for rowwise output, a
// column for columnwise output) draws byte i % 16 of Philox block
// (i / 16, vector, direction, offset) under key (k0, k1), direction 0
// rowwise, 1 columnwise, the block's words read as little-endian bytes.  A
// lane holds a 16-row x 8-column sub-block (as in the deterministic cast); a
// workgroup covers 128 rows x 256 columns.  Per-token outer scales are
// computed once per workgroup into LDS; rows go two at a time, the lane pair
// splitting their block parameters (the even lane the even row's, the odd
// lane the odd row's, handed across by DPP) and their Philox blocks (the
// even lane draws the even row's block, whose 16 bytes cover both lanes'
// columns, the odd lane the odd row's; each hands the other the two words it
// needs).  A column's 16 rows take one block.  Built for
// four waves per SIMD (at most 128 VGPRs; one 8-byte value spills, outside
// the element loops): the Philox rounds are chains of dependent operations
// that more waves hide better.  Requires M < 2^32 (the vector index is one
// counter word).
template <int MODE, bool ROW, bool COL>
__global__ __launch_bounds__(256, 4) void k_encode_sr(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                   const float* __restrict__ row_amax, const float* __restrict__ col_amax,
                                                   uint8_t* __restrict__ row_q, uint8_t* __restrict__ row_sf,
                                                   uint8_t* __restrict__ col_q, uint8_t* __restrict__ col_sf,
                                                   uint32_t k0, uint32_t k1, uint32_t offset) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, rg = lane >> 5;
    const bool odd = lane & 1;
    const uint32_t tc0 = blockIdx.x * kEncCols;
    const int64_t tr0 = (int64_t)blockIdx.y * 128;
    const uint32_t c0 = tc0 + (lane & 31) * 8;
    const int rl0 = wave * 32 + 16 * rg;   // the lane's first row within the tile
    const int64_t r0 = tr0 + rl0;
    const bool col_ok = c0 < K;
    const int nrows = r0 >= M ? 0 : (M - r0 < 16 ? (int)(M - r0) : 16);
    auto load_row = [&](int i) {
        return (col_ok && i < nrows) ? *reinterpret_cast<const u32x4*>(x + (r0 + i) * K + c0) : u32x4{0u, 0u, 0u, 0u};
    };
    constexpr bool TOK = MODE == ENC_TOKEN;
    __shared__ float2 rsc[(TOK && ROW) ? 128 : 1];
    __shared__ float2 csc[(TOK && COL) ? kEncCols : 1];
    if (TOK) {
        const int t = threadIdx.x;
        if (COL) csc[t] = outer_entry(tc0 + t < K ? col_amax[tc0 + t] : 0.0f);
        if (ROW && t < 128) rsc[t] = outer_entry(tr0 + t < M ? row_amax[tr0 + t] : 0.0f);
        __syncthreads();
    }
    if (ROW) {
        const Outer rot = make_outer(TOK ? 0.0f : row_amax[0]);
        const uint32_t own_sel = odd ? 0x03020c0cu : 0x01000c0cu;   // own row's half to the top
        // rows two at a time (a rolled loop: unrolled, its register arrays
        // would go to scratch memory), the next pair's loads issued before
        // this pair is encoded
        u32x4 n0 = load_row(0), n1 = load_row(1);
#pragma unroll 1
        for (int i = 0; i < 16; i += 2) {
            const u32x4 w0 = n0, w1 = n1;
            if (i + 2 < 16) {
                n0 = load_row(i + 2);
                n1 = load_row(i + 3);
            }
            const uint32_t rw0 = rowmax_word(w0), rw1 = rowmax_word(w1);
            // (row i | row i+1 << 16) over the lane's 8 columns, then the pair's 16
            uint32_t m = pk_max_u16(__builtin_amdgcn_perm(rw1, rw0, 0x05040100u),
                                    __builtin_amdgcn_perm(rw1, rw0, 0x07060302u));
            m = pk_max_u16(m, from_pair(m));
            const Outer ro = TOK ? outer_from(rsc[rl0 + i + (odd ? 1 : 0)]) : rot;
            const SrBlock f = sr_block(__builtin_amdgcn_perm(m, m, own_sel), ro);
            const bool fast = __builtin_amdgcn_ballot_w64(f.slow) == 0ull;
            const float rr0 = from_even(f.r), ry0 = from_even(f.y), rr1 = from_odd(f.r), ry1 = from_odd(f.y);
            BlockScale b0, b1;
            if (!fast) {
                const float A0 = TOK ? (i < nrows ? row_amax[r0 + i] : 0.0f) : row_amax[0];
                const float A1 = TOK ? (i + 1 < nrows ? row_amax[r0 + i + 1] : 0.0f) : row_amax[0];
                b0 = block_scale(m & 0xffffu, outer_scale(A0));
                b1 = block_scale(m >> 16, outer_scale(A1));
            }
            // the pair's randoms: the lane's columns c0 .. c0+7 are bytes
            // (c0 % 16) .. +7, two words, of each row's block (c0 / 16, row)
            const u32x4 P = philox4x32_10(c0 >> 4, (uint32_t)(r0 + i + (odd ? 1 : 0)), 0u, offset, k0, k1);
            const uint32_t t0 = from_pair(odd ? P.x : P.z), t1 = from_pair(odd ? P.y : P.w);
            const uint32_t rw[2][2] = {{odd ? t0 : P.x, odd ? t1 : P.y}, {odd ? P.z : t0, odd ? P.w : t1}};
            uint32_t wq[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32x4 vi = h ? w1 : w0;
                const uint32_t g0 = rw[h][0], g1 = rw[h][1];
                float qv[8];
                if (fast) {
                    const float r = h ? rr1 : rr0, y = h ? ry1 : ry0;
#pragma unroll
                    for (int k = 0; k < 8; ++k) qv[k] = div_fast(elem(vi, k), r, y);
                } else {
                    const BlockScale& bs = h ? b1 : b0;
#pragma unroll
                    for (int k = 0; k < 8; ++k) qv[k] = quotient_exact(elem(vi, k), bs);
                }
                wq[h] = e2m1_sr8<0>(qv[0], g0, g1) | e2m1_sr8<1>(qv[1], g0, g1) << 4 |
                        e2m1_sr8<2>(qv[2], g0, g1) << 8 | e2m1_sr8<3>(qv[3], g0, g1) << 12 |
                        e2m1_sr8<4>(qv[4], g0, g1) << 16 | e2m1_sr8<5>(qv[5], g0, g1) << 20 |
                        e2m1_sr8<6>(qv[6], g0, g1) << 24 | e2m1_sr8<7>(qv[7], g0, g1) << 28;
            }
            const uint32_t code = fast ? f.code : (odd ? b1.code : b0.code);
            if (col_ok) {
                // a row's 32 lanes write one whole 128-byte line: nontemporal
                if (i < nrows) __builtin_nontemporal_store(wq[0], reinterpret_cast<uint32_t*>(row_q + (r0 + i) * (K / 2) + c0 / 2));
                if (i + 1 < nrows) __builtin_nontemporal_store(wq[1], reinterpret_cast<uint32_t*>(row_q + (r0 + i + 1) * (K / 2) + c0 / 2));
                const int io = i + (odd ? 1 : 0);
                if (io < nrows) row_sf[(r0 + io) * (K / 16) + c0 / 16] = (uint8_t)code;
            }
        }
    }
    if (COL) {
        u32x4 v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = load_row(i);
        const Outer cot = make_outer(TOK ? 0.0f : col_amax[0]);
#pragma unroll 1
        for (int j = 0; j < 8; ++j) {
            uint32_t m = 0u;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t e = (__float_as_uint(elem_rt(v[i], j)) >> 16) & 0x7fffu;
                m = e > m ? e : m;
            }
            const Outer co = TOK ? outer_from(csc[(lane & 31) * 8 + j]) : cot;
            const SrBlock f = sr_block(m << 16, co);
            // the column's 16 rows take bytes 0..15 of one block (r0 / 16, column)
            const u32x4 P = philox4x32_10((uint32_t)(r0 >> 4), c0 + (uint32_t)j, 1u, offset, k0, k1);
            const uint32_t rr[4] = {P.x, P.y, P.z, P.w};
            uint32_t lohi[2] = {0u, 0u};
            uint32_t code;
            // one element at a time (the empty asm): the rounding has no
            // branches, and sixteen of it in flight would cost registers
            auto col_codes = [&](auto quot) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    lohi[g >> 1] |= e2m1_sr<0>(quot(4 * g), rr[g]) << (4 * ((4 * g) & 7));
                    asm volatile("" : "+v"(lohi[0]), "+v"(lohi[1]));
                    lohi[g >> 1] |= e2m1_sr<1>(quot(4 * g + 1), rr[g]) << (4 * ((4 * g + 1) & 7));
                    asm volatile("" : "+v"(lohi[0]), "+v"(lohi[1]));
                    lohi[g >> 1] |= e2m1_sr<2>(quot(4 * g + 2), rr[g]) << (4 * ((4 * g + 2) & 7));
                    asm volatile("" : "+v"(lohi[0]), "+v"(lohi[1]));
                    lohi[g >> 1] |= e2m1_sr<3>(quot(4 * g + 3), rr[g]) << (4 * ((4 * g + 3) & 7));
                    asm volatile("" : "+v"(lohi[0]), "+v"(lohi[1]));
                }
            };
            if (__builtin_amdgcn_ballot_w64(f.slow) == 0ull) {
                code = f.code;
                col_codes([&](int i) { return div_fast(elem_rt(v[i], j), f.r, f.y); });
            } else {
                const float A = TOK ? (col_ok ? col_amax[c0 + j] : 0.0f) : col_amax[0];
                const BlockScale bs = block_scale(m, outer_scale(A));
                code = bs.code;
                col_codes([&](int i) { return quotient_exact(elem_rt(v[i], j), bs); });
            }
            if (col_ok && nrows == 16) {
                *reinterpret_cast<u32x2*>(col_q + (int64_t)(c0 + j) * (M / 2) + r0 / 2) = u32x2{lohi[0], lohi[1]};
                col_sf[(int64_t)(c0 + j) * (M / 16) + r0 / 16] = (uint8_t)code;
            }
        }
    }
}

// ---------------------------------------------------------------- dequantize

// one thread per 16-element block: out = (+/-) g * (decode(sf) * (A / 2688)),
// fp32, or (BF16) that fp32 value rounded to nearest-even bf16
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;   // finite inputs (NaN cannot arise here)
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ q, const uint8_t* __restrict__ sf,
                                                 const float* __restrict__ amax, int64_t R, int64_t C,
                                                 int amax_per_row, void* __restrict__ out) {
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
        if (BF16) {
            uint32_t h[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) h[i] = bf16_rne(o[2 * i]) | (bf16_rne(o[2 * i + 1]) << 16);
            u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + r * C + 16 * j);
            dst[0] = u32x4{h[0], h[1], h[2], h[3]};
            dst[1] = u32x4{h[4], h[5], h[6], h[7]};
        } else {
            float4* dst = reinterpret_cast<float4*>(static_cast<float*>(out) + r * C + 16 * j);
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
        }
    }
}

// ------------------------------------------------ resident one-launch cast
//
// Per-tensor and per-token casts whose amax is measured on x, in a single
// launch of at most one workgroup per compute unit, all resident at once.
// Phase A reads the workgroup's tiles and combines their maxima into the
// amax outputs (zeroed first, as in the amax pass); then a grid-wide wait;
// phase B encodes.  The last two tiles a wave reads in phase A stay in its
// registers and are encoded in phase B without a second read: a tensor of at
// most two tiles per workgroup crosses HBM once, a larger one re-reads the
// rest (nontemporal, most recently read first).  With two waves per SIMD
// and all of the cast's vector work in phase B, runs longer than two tiles
// are slower than the two-launch schedule; the host uses this kernel for
// them only when asked to.
//
// Work: 256-row x 256-column tiles.  Workgroup w (8 waves) owns a vertical
// run of up to `run` tiles of strip w / nband (256 columns), band w % nband
// (so the strips of a band share an XCD when nband % 8 == 0, and write the
// same rowwise scale lines through one L2).  Its column maxima accumulate in
// registers over the run and the strip's column scales are set once in
// phase B.  Wave v covers rows 32v .. 32v+31 of each tile, laid out as a
// step of the encode pass (two 32-lane row groups, a 16-row x 8-column
// sub-block per lane).
//
// Phase A walks the run from its last tile down: tile t sits in register set
// t % 2, and tile t - 2 is loaded into that set once tile t's maxima are
// taken.  Phase B walks up from tile 0 and loads tile t + 2 into the set of
// tile t as that one is encoded.  Phase B reads the amax outputs with
// coherent (atomic) loads: the grid-wide wait carries no acquire, and a
// cache may still hold the zeros written before phase A.

__device__ __forceinline__ float load_coherent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Max over each 32-lane half of the wave of 16 per-lane 16-bit values (one
// per row), by halving exchanges: after the xor-16/8/4 steps each lane holds
// a pair of rows, the xor-2/1 steps finish.  Returns the pair index j (rows
// 2j, 2j+1 in the low / high half of *pair) this lane holds.
__device__ __forceinline__ int half_rowmax16(const uint32_t m[16], uint32_t* pair) {
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

// wg_accumulate_reduce over amax values other workgroups of the same launch
// combined: obs is read with coherent loads
__device__ void wg_accumulate_reduce_coherent(float* __restrict__ buf, const float* obs, int64_t n, float decay,
                                              float* red) {
    float m = 0.0f;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
        const float o = load_coherent(obs + i);
        m = o > m ? o : m;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const float o = __shfl_xor(m, d);
        m = o > m ? o : m;
    }
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        const int nw = (int)(blockDim.x >> 6);
        for (int w = 1; w < nw; ++w) m = red[w] > m ? red[w] : m;
        const float t = buf[0] * decay;
        buf[0] = m > t ? m : t;
    }
}

template <int MODE, bool ROW, bool COL>
__global__ __launch_bounds__(512) void k_resident(ResArgs a) {
    constexpr bool TOK = MODE == ENC_TOKEN;
    constexpr bool ROWTOK = ROW && TOK;
    constexpr bool COL_LDS = COL && TOK;
    __shared__ float row_scale[8][32][2];    // per wave: S and 1/S of the step's 32 rows
    __shared__ float2 col_scale[COL_LDS ? kEncCols : 1];
    __shared__ uint32_t red[8][32][4];
    __shared__ int bar_ok;
    // per-token rowwise: the amax of the band's rows, read once after the
    // grid-wide wait (LDS reads in the steps keep memory waits for x alone)
    __shared__ float band_amax[ROWTOK ? kResMaxRun * kEncRows : 1];

    const uint16_t* __restrict__ x = a.x;
    const int64_t M = a.M, K = a.K;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lin = blockIdx.x;
    const uint32_t strip = lin / (uint32_t)a.nband, band = lin % (uint32_t)a.nband;
    const int64_t ty = (M + kEncRows - 1) / kEncRows;
    const int64_t t_first = (int64_t)band * a.run;
    const int tcount = (int)(ty - t_first < a.run ? ty - t_first : a.run);   // >= 1
    const int rg = lane >> 5;
    const uint32_t c0 = strip * kEncCols + (lane & 31) * 8;
    const bool col_ok = c0 < K;
    const bool odd = lane & 1;
    const uint32_t xrow = (uint32_t)K * 2u, qrow = (uint32_t)(K / 2), srow = (uint32_t)(K / 16);
    const uint32_t vx = col_ok ? 16u * rg * xrow + c0 * 2u : kOffOut;
    auto tile_r0 = [&](int t) -> int64_t { return (t_first + t) * kEncRows; };
    // valid rows of the wave's step of tile t (0 outside the run)
    auto step_rows = [&](int t) -> uint32_t {
        if (t < 0 || t >= tcount) return 0u;
        const int64_t left = M - (tile_r0(t) + 32 * wave);
        return left <= 0 ? 0u : (left < 32 ? (uint32_t)left : 32u);
    };
    auto x_rsrc = [&](int t) {
        const uint32_t n = step_rows(t);
        return n ? rsrc(x + (tile_r0(t) + 32 * wave) * K, n * xrow) : rsrc(x, 0u);
    };

    // Zero-first as in the amax pass, but with device-scope stores (performed
    // beyond the caches, like the atomics that follow) and a relaxed arrival
    // once they are complete: a release here would write back the whole L2.
    const bool zon = a.zsync.slot >= 0;
    if (zon && lin < (uint32_t)a.zero.wgs) {
        const int64_t z0 = (int64_t)lin * kZeroPerWg, z1 = z0 + kZeroPerWg;
        for (int64_t i = z0 + threadIdx.x; i < z1 && i < a.zero.na + a.zero.nb; i += blockDim.x) {
            float* p = i < a.zero.na ? a.zero.a + i : a.zero.b + (i - a.zero.na);
            __hip_atomic_store(p, 0.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) sync_arrive_relaxed(a.zsync);
    }
    // Phase A's atomics all come after its loop, behind one wait for the
    // zeroing workgroups (one lane polls for the workgroup).  Until then the
    // per-token row-pair maxima of each tile and wave sit in LDS, in the
    // space band_amax takes after the grid-wide wait: entry (t * 8 + wave) *
    // 16 + e holds rows 16 (e >> 3) + 2 (e & 7) and the next of the wave's 32.
    __shared__ int zero_ok;
    uint32_t* const rowred = reinterpret_cast<uint32_t*>(band_amax);
    static_assert(!ROWTOK || kResMaxRun * kEncRows >= kResMaxRun * 8 * 16, "row-pair maxima fit in band_amax");

    uint32_t xr = xrow;
    asm volatile("" : "+s"(xr));   // keeps the 16 row offsets out of vector registers

    // ---------------------------------------------------------- phase A
    u32x4 v0[16], v1[16];
    uint32_t cm[4] = {0u, 0u, 0u, 0u};   // column maxima over the run (columns 2k | 2k+1 << 16)
    uint32_t tm = 0u;                    // tensor maximum (two halves)
    const int tpad = (tcount + 1) & ~1;
    {
        const __amdgpu_buffer_rsrc_t r1 = x_rsrc(tpad - 1), r0 = x_rsrc(tpad - 2);
#pragma unroll
        for (int i = 0; i < 16; ++i) v1[i] = __builtin_amdgcn_raw_buffer_load_b128(r1, vx, i * xr, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) v0[i] = __builtin_amdgcn_raw_buffer_load_b128(r0, vx, i * xr, 0);
    }
    // (load: tile t - 2 follows into v; false for the kept tiles 0 and 1)
    auto amax_step = [&](u32x4(&v)[16], int t, bool load) {
        const __amdgpu_buffer_rsrc_t nrs = x_rsrc(t - 2);
        uint32_t rm[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t a0 = abs2(v[i].x), a1 = abs2(v[i].y), a2 = abs2(v[i].z), a3 = abs2(v[i].w);
            if (COL && TOK) {
                cm[0] = pk_max_u16(cm[0], a0);
                cm[1] = pk_max_u16(cm[1], a1);
                cm[2] = pk_max_u16(cm[2], a2);
                cm[3] = pk_max_u16(cm[3], a3);
            }
            const uint32_t r = pk_max_u16(pk_max_u16(a0, a1), pk_max_u16(a2, a3));
            if (TOK) rm[i] = max_halves(r);
            else tm = pk_max_u16(tm, r);
            if (load) {
                uint32_t so = i * xr;
                asm volatile("" : "+s"(so) : "v"(r), "v"(cm[0]), "v"(cm[1]), "v"(cm[2]), "v"(cm[3]), "v"(tm));
                v[i] = __builtin_amdgcn_raw_buffer_load_b128(nrs, vx, so, 0);
            }
        }
        if (ROWTOK && t < tcount) {
            uint32_t pair;
            half_rowmax16(rm, &pair);   // lane 4e: pair e & 7 of row group e >> 3
            if ((lane & 3) == 0) rowred[(t * 8 + wave) * 16 + (lane >> 2)] = pair;
        }
    };
    // The memory-wait counts the compiler derives across the loop's back
    // edge are exact only when every pass issues the same loads: the last
    // pair, which loads nothing, is peeled off.
#pragma unroll 1
    for (int t = tpad - 2; t >= 2; t -= 2) {
        amax_step(v1, t + 1, true);
        amax_step(v0, t, true);
    }
    amax_step(v1, 1, false);
    amax_step(v0, 0, false);
    if (COL && TOK) {
#pragma unroll
        for (int k = 0; k < 4; ++k) cm[k] = pk_max_u16(cm[k], (uint32_t)__shfl_xor((int)cm[k], 32));
        if (lane < 32) {
#pragma unroll
            for (int k = 0; k < 4; ++k) red[wave][lane][k] = cm[k];
        }
    }
    if (!TOK) {
        const uint32_t w = wave_max(max_halves(tm));
        if (lane == 0) red[wave][0][0] = w;
    }
    if (threadIdx.x == 0) zero_ok = !zon || sync_poll(a.zsync, (unsigned long long)a.zero.wgs);
    __syncthreads();
    // (a workgroup whose wait gave up skips the atomics but still arrives
    // at the grid-wide wait below)
    if (ROWTOK && zero_ok) {
        for (int i = threadIdx.x; i < tcount * 128; i += blockDim.x) {
            const int t = i >> 7, w = (i >> 4) & 7, e = i & 15;
            const uint32_t pair = rowred[i];
            const int64_t r = tile_r0(t) + 32 * w + 16 * (e >> 3) + 2 * (e & 7);
            if (r < M) atomic_max_mag(a.row_amax + r, pair & 0xffffu);
            if (r + 1 < M) atomic_max_mag(a.row_amax + r + 1, pair >> 16);
        }
    }
    if (COL && TOK) {
        // one atomic per column: threads 0..127 take a column pair each
        if (wave < 2 && zero_ok) {
            const int l = threadIdx.x >> 2, k = threadIdx.x & 3;
            uint32_t m = 0u;
#pragma unroll
            for (int w = 0; w < 8; ++w) m = pk_max_u16(m, red[w][l][k]);
            const uint32_t c = strip * kEncCols + l * 8 + 2 * k;
            if (c < K) {
                atomic_max_mag(a.col_amax + c, m & 0xffffu);
                atomic_max_mag(a.col_amax + c + 1, m >> 16);
            }
        }
    }
    if (!TOK && threadIdx.x == 0 && zero_ok) {
        uint32_t m = 0u;
        for (int w = 0; w < 8; ++w) m = m > red[w][0][0] ? m : red[w][0][0];
        if (ROW) atomic_max_mag(a.row_amax, m);
        if (COL) atomic_max_mag(a.col_amax, m);
    }

    // ------------------------------------------------ grid-wide wait
    // Every wave's atomics are complete before its workgroup arrives (they
    // are performed beyond the caches, so no release is needed: one would
    // write back the whole L2, per workgroup).
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) bar_ok = sync_grid_wait(a.bar, gridDim.x, lin) ? 1 : 0;
    __syncthreads();
    if (!bar_ok) return;

    // ---------------------------------------------------------- phase B
    // outer scales: the strip's columns (per token, in LDS) or the tensor's
    // (all loads issued before any is used: one memory round trip)
    bool col_slow = false;
    float rowA_t = 0.0f, colA_t = 0.0f;
    Outer rowO_t{1.0f, 1.0f, false}, colO_t{1.0f, 1.0f, false};
    {
        const uint32_t c = strip * kEncCols + (threadIdx.x & (kEncCols - 1));
        const float ca = (COL_LDS && threadIdx.x < kEncCols && c < K) ? load_coherent(a.col_amax + c) : 0.0f;
        constexpr int kPer = ROWTOK ? kResMaxRun * kEncRows / 512 : 1;
        float ba[kPer];
        const int64_t b0 = tile_r0(0);
        const int64_t nb = M - b0 < (int64_t)tcount * kEncRows ? M - b0 : (int64_t)tcount * kEncRows;
        if (ROWTOK) {
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                const int64_t i = threadIdx.x + 512 * k;
                ba[k] = i < nb ? load_coherent(a.row_amax + b0 + i) : 0.0f;
            }
        }
        if (!TOK) {
            if (ROW) rowA_t = load_coherent(a.row_amax);
            if (COL) colA_t = load_coherent(a.col_amax);
        }
        bool sl = false;
        if (COL_LDS && threadIdx.x < kEncCols) {
            const Outer o = make_outer(ca, c < K);
            col_scale[threadIdx.x] = make_float2(o.S, o.yS);
            sl = o.slow;
        }
        if (ROWTOK) {
#pragma unroll
            for (int k = 0; k < kPer; ++k)
                if (threadIdx.x + 512 * k < nb) band_amax[threadIdx.x + 512 * k] = ba[k];
        }
        col_slow = __syncthreads_or(sl) != 0;
    }
    if (!TOK) {
        rowO_t = make_outer(rowA_t, ROW);
        colO_t = make_outer(colA_t, COL);
    }
    const bool tensor_slow = !TOK && ((ROW && rowO_t.slow) || (COL && colO_t.slow));
    // the calibration update: one workgroup reduces the finished amax
    if (a.cal.buf != nullptr && lin == 0u) {
        wg_accumulate_reduce_coherent(a.cal.buf, a.cal.obs, a.cal.n, a.cal.decay, &row_scale[0][0][0]);
        __syncthreads();
    }

    const uint32_t vq = col_ok ? 16u * rg * qrow + c0 / 2u : kOffOut;
    const uint32_t vs = col_ok ? (16u * rg + (odd ? 1u : 0u)) * srow + c0 / 16u : kOffOut;
    const uint32_t own_sel = odd ? 0x03020c0cu : 0x01000c0cu;
    uint32_t slow_mask = 0u;   // tiles of the run this wave must encode again (run <= 32)

    // Columnwise output goes straight to memory (no LDS staging, so phase B
    // has no workgroup barrier): a lane's 8 columns x 16 rows are 8 bytes of
    // data and one scale byte per column; the lane part of each offset is
    // fixed, the tile and column parts are scalar.  Lanes l and l + 32 write
    // adjacent halves of 16 bytes, the 8 waves a tile's 128 bytes of each
    // column, merged in the L2 (ordinary stores: nontemporal ones reach
    // memory in pieces and measured slower).
    const __amdgpu_buffer_rsrc_t cq_rs = rsrc(a.col_q, COL ? (uint32_t)(M / 2 * K) : 0u);
    const __amdgpu_buffer_rsrc_t cs_rs = rsrc(a.col_sf, COL ? (uint32_t)(M / 16 * K) : 0u);
    const uint32_t vcq = col_ok ? c0 * (uint32_t)(M / 2) + (32u * wave + 16u * rg) / 2u : kOffOut;
    const uint32_t vcs = col_ok ? c0 * (uint32_t)(M / 16) + (32u * wave + 16u * rg) / 16u : kOffOut;
    const uint32_t mq = (uint32_t)(M / 2), ms = (uint32_t)(M / 16);

    auto enc_step = [&](u32x4(&v)[16], int t) {
        const int64_t wr0 = tile_r0(t) + 32 * wave;
        const uint32_t nrows = step_rows(t);
        const bool group_ok = 16u * rg < nrows;
        const int64_t r0 = group_ok ? wr0 + 16 * rg : wr0;
        uint32_t qr = qrow, sr = srow;
        asm volatile("" : "+s"(qr), "+s"(sr));
        SubDst d;
        d.row_q = a.row_q + r0 * (K / 2);
        d.row_sf = a.row_sf + r0 * (K / 16);
        d.col_q = nullptr;
        d.col_sf = nullptr;
        d.row_q_stride = qrow;
        d.row_sf_stride = srow;
        d.col_q_stride = (uint32_t)(M / 2);
        d.col_sf_stride = (uint32_t)(M / 16);
        d.c0 = c0;
        d.nrows = group_ok ? (int)(nrows - 16u * rg < 16u ? nrows - 16u * rg : 16u) : 0;
        d.col_ok = col_ok && group_ok;
        d.odd = odd;
        d.lds_q = nullptr;
        d.lds_sf = nullptr;
        // the sub-block's columnwise offsets (16-row groups past the end store nothing)
        const uint32_t tq = (uint32_t)(tile_r0(t) / 2), ts = (uint32_t)(tile_r0(t) / 16);
        const uint32_t lq = group_ok ? vcq : kOffOut, ls = group_ok ? vcs : kOffOut;

        // rowwise outer scales of the step's rows: lanes 0..31 one row each
        bool step_slow = tensor_slow;
        if (ROWTOK) {
            const bool row_in = (uint32_t)(lane & 31) < nrows;
            const Outer o = make_outer(row_in ? band_amax[t * kEncRows + 32 * wave + (lane & 31)] : 0.0f, row_in);
            if (lane < 32) {
                row_scale[wave][lane][0] = o.S;
                row_scale[wave][lane][1] = o.yS;
            }
            step_slow |= __builtin_amdgcn_ballot_w64(o.slow) != 0ull;
            // other lanes read these entries below: keep the reads after the writes
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }

        // maxima from the packed words
        bool slow = col_slow;
        uint32_t bcm[4] = {0u, 0u, 0u, 0u};   // column block maxima (columns 2k | 2k+1 << 16)
        uint32_t bm[8];                        // rowwise block max of the own row of pair s
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            uint32_t rw[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32x4 w = v[2 * s + h];
                const uint32_t a0 = abs2(w.x), a1 = abs2(w.y), a2 = abs2(w.z), a3 = abs2(w.w);
                if (COL) {
                    bcm[0] = pk_max_u16(bcm[0], a0);
                    bcm[1] = pk_max_u16(bcm[1], a1);
                    bcm[2] = pk_max_u16(bcm[2], a2);
                    bcm[3] = pk_max_u16(bcm[3], a3);
                }
                rw[h] = pk_max_u16(pk_max_u16(a0, a1), pk_max_u16(a2, a3));
            }
            if (ROW) {
                uint32_t m = pk_max_u16(__builtin_amdgcn_perm(rw[1], rw[0], 0x05040100u),
                                        __builtin_amdgcn_perm(rw[1], rw[0], 0x07060302u));
                m = pk_max_u16(m, from_pair(m));
                bm[s] = __builtin_amdgcn_perm(m, m, own_sel);
            }
        }
        if (ROW)
            asm volatile("" : "+v"(bm[0]), "+v"(bm[1]), "+v"(bm[2]), "+v"(bm[3]),
                         "+v"(bm[4]), "+v"(bm[5]), "+v"(bm[6]), "+v"(bm[7]));
        FastBlock cb[8];
        if (COL) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t bits = (j & 1) ? (bcm[j >> 1] & 0xffff0000u) : (bcm[j >> 1] << 16);
                Outer o = colO_t;
                if (COL_LDS) {
                    const float2 sy = col_scale[(lane & 31) * 8 + j];
                    o.S = sy.x;
                    o.yS = sy.y;
                }
                cb[j] = fast_block<false, true>(bits, o);
                slow |= cb[j].slow;
                __builtin_amdgcn_raw_buffer_store_b8((uint8_t)cb[j].code, cs_rs, ls, ts + j * ms, 0);
            }
        }

        // per row pair: rowwise parameters, then both encodings
        const __amdgpu_buffer_rsrc_t q_rs = rsrc(a.row_q + wr0 * (K / 2), nrows * qrow);
        const __amdgpu_buffer_rsrc_t s_rs = rsrc(a.row_sf + wr0 * (K / 16), nrows * srow);
        uint32_t cq[8][2] = {};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int i = 2 * s;
            float yh0 = 0.0f, yl0 = 0.0f, yh1 = 0.0f, yl1 = 0.0f;
            if (ROW) {
                Outer ro = rowO_t;
                if (ROWTOK) {
                    ro.S = row_scale[wave][16 * rg + i + (odd ? 1 : 0)][0];
                    ro.yS = row_scale[wave][16 * rg + i + (odd ? 1 : 0)][1];
                }
                const FastBlock f = fast_block<false, true>(bm[s], ro);
                slow |= f.slow;
                __builtin_amdgcn_raw_buffer_store_b8((uint8_t)f.code, s_rs, vs, i * sr, 0);
                yh0 = from_even(f.yh); yl0 = from_even(f.yl);
                yh1 = from_odd(f.yh);  yl1 = from_odd(f.yl);
            }
            // pair s is unpacked only after pair s-1's outputs are done
            u32x4 w0 = v[i], w1 = v[i + 1];
            if (COL && s > 0)
                asm volatile("" : "+v"(w0), "+v"(w1), "+v"(cq[0][(s - 1) >> 2]), "+v"(cq[1][(s - 1) >> 2]),
                             "+v"(cq[2][(s - 1) >> 2]), "+v"(cq[3][(s - 1) >> 2]), "+v"(cq[4][(s - 1) >> 2]),
                             "+v"(cq[5][(s - 1) >> 2]), "+v"(cq[6][(s - 1) >> 2]), "+v"(cq[7][(s - 1) >> 2]));
            else
                asm volatile("" : "+v"(w0), "+v"(w1));
            const float a0[8] = {bf_lo(w0.x), bf_hi(w0.x), bf_lo(w0.y), bf_hi(w0.y),
                                 bf_lo(w0.z), bf_hi(w0.z), bf_lo(w0.w), bf_hi(w0.w)};
            const float a1[8] = {bf_lo(w1.x), bf_hi(w1.x), bf_lo(w1.y), bf_hi(w1.y),
                                 bf_lo(w1.z), bf_hi(w1.z), bf_lo(w1.w), bf_hi(w1.w)};
            if (COL) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float q0 = quot2(a0[j], cb[j].yh, cb[j].yl), q1 = quot2(a1[j], cb[j].yh, cb[j].yl);
                    uint32_t& w = cq[j][s >> 2];
                    if ((s & 3) == 0) w = put_fp4x2<0>(__float_as_uint(q0), q0, q1);
                    else if ((s & 3) == 1) w = put_fp4x2<1>(w, q0, q1);
                    else if ((s & 3) == 2) w = put_fp4x2<2>(w, q0, q1);
                    else w = put_fp4x2<3>(w, q0, q1);
                }
            }
            uint32_t o0 = 0u, o1 = 0u;
            if (ROW) {
                const float p00 = quot2(a0[0], yh0, yl0), p10 = quot2(a1[0], yh1, yl1);
                o0 = put_fp4x2<0>(__float_as_uint(p00), p00, quot2(a0[1], yh0, yl0));
                o0 = put_fp4x2<1>(o0, quot2(a0[2], yh0, yl0), quot2(a0[3], yh0, yl0));
                o0 = put_fp4x2<2>(o0, quot2(a0[4], yh0, yl0), quot2(a0[5], yh0, yl0));
                o0 = put_fp4x2<3>(o0, quot2(a0[6], yh0, yl0), quot2(a0[7], yh0, yl0));
                o1 = put_fp4x2<0>(__float_as_uint(p10), p10, quot2(a1[1], yh1, yl1));
                o1 = put_fp4x2<1>(o1, quot2(a1[2], yh1, yl1), quot2(a1[3], yh1, yl1));
                o1 = put_fp4x2<2>(o1, quot2(a1[4], yh1, yl1), quot2(a1[5], yh1, yl1));
                o1 = put_fp4x2<3>(o1, quot2(a1[6], yh1, yl1), quot2(a1[7], yh1, yl1));
                __builtin_amdgcn_raw_buffer_store_b32(o0, q_rs, vq, i * qr, kCacheNT);
                __builtin_amdgcn_raw_buffer_store_b32(o1, q_rs, vq, (i + 1) * qr, kCacheNT);
            }
        }
        if (COL) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{cq[j][0], cq[j][1]}, cq_rs, lq, tq + j * mq, 0);
        }
        // a block outside the fast path's range: the sub-block is encoded
        // again, exactly, after the last tile
        if ((step_slow || __builtin_amdgcn_ballot_w64(slow) != 0ull) && t < tcount) slow_mask |= 1u << t;
        // tile t + 2 into this register set, encoded two steps on (past the
        // run: an empty buffer, zeros without a memory access; issued either
        // way so that every step issues the same loads)
        {
            const __amdgpu_buffer_rsrc_t nx_rs = x_rsrc(t + 2);
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(nx_rs, vx, i * xr, kCacheNT);
        }
        // the next step's row scales overwrite entries other lanes read above
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    };

    // whole pairs in the loop (every pass issues the same loads), then the
    // odd tile
#pragma unroll 1
    for (int t = 0; t + 1 < tcount; t += 2) {
        enc_step(v0, t);
        enc_step(v1, t + 1);
    }
    if (tcount & 1) enc_step(v0, tcount - 1);

    // Exact pass over the flagged steps (by the lanes that stored them: a
    // wave's stores to one address land in order).
    while (slow_mask != 0u) {
        const int t = __builtin_ctz(slow_mask);
        slow_mask &= slow_mask - 1u;
        const uint32_t nrows = step_rows(t);
        const bool group_ok = 16u * rg < nrows;
        const int64_t r0 = tile_r0(t) + 32 * wave + (group_ok ? 16 * rg : 0);
        SubDst d;
        d.row_q = a.row_q + r0 * (K / 2);
        d.row_sf = a.row_sf + r0 * (K / 16);
        d.col_q = a.col_q + r0 / 2;
        d.col_sf = a.col_sf + r0 / 16;
        d.row_q_stride = qrow;
        d.row_sf_stride = srow;
        d.col_q_stride = (uint32_t)(M / 2);
        d.col_sf_stride = (uint32_t)(M / 16);
        d.c0 = c0;
        d.nrows = group_ok ? (int)(nrows - 16u * rg < 16u ? nrows - 16u * rg : 16u) : 0;
        d.col_ok = col_ok && group_ok;
        d.odd = odd;
        d.lds_q = nullptr;
        d.lds_sf = nullptr;
        float rowA[16], colA[8];
        for (int i = 0; i < 16; ++i)
            rowA[i] = !ROW ? 0.0f : !TOK ? rowA_t : (i < d.nrows ? load_coherent(a.row_amax + r0 + i) : 0.0f);
        for (int j = 0; j < 8; ++j)
            colA[j] = !COL ? 0.0f : !TOK ? colA_t : (col_ok ? load_coherent(a.col_amax + c0 + j) : 0.0f);
        encode_exact<ROW, COL, false, false, false>(x + r0 * K, K, rowA, colA, 0.0f, d);
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

__global__ __launch_bounds__(1024) void k_accumulate_reduce(float* __restrict__ buf, const float* __restrict__ obs,
                                                            int64_t n, float decay) {
    __shared__ float red[16];
    wg_accumulate_reduce(buf, obs, n, decay, red);
}

// ------------------------------------------------------------------ launchers

static inline unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

hipError_t launch_fill2(float* p, int64_t n, float* q, int64_t m, float v, hipStream_t st) {
    if (p == nullptr) n = 0;
    if (q == nullptr) m = 0;
    if (n + m <= 0) return hipSuccess;
    unsigned grid = cdiv(n + m, 256);
    if (grid > 4096) grid = 4096;
    hipLaunchKernelGGL(k_fill2_u32, dim3(grid), dim3(256), 0, st, reinterpret_cast<uint32_t*>(p), n,
                       reinterpret_cast<uint32_t*>(q), m, __builtin_bit_cast(uint32_t, v));
    return hipGetLastError();
}

// rows per workgroup of the amax pass: 512 (256 for grouped casts), fewer
// when the grid would leave CUs idle
static int amax_tile_h(int kind, int64_t K, int64_t row_begin, int64_t row_end) {
    int tile_h = kAmaxRows;
    while (tile_h > 64 && (int64_t)cdiv(K, kTileCols) * cdiv(row_end - row_begin, tile_h) < 512) tile_h /= 2;
    if (kind == AMAX_GROUPED && tile_h > kAmaxGroupedRows) tile_h = kAmaxGroupedRows;
    return tile_h;
}

int64_t amax_grid_size(int kind, int64_t K, int64_t row_begin, int64_t row_end) {
    if (row_end <= row_begin || K <= 0) return 0;
    return (int64_t)cdiv(K, kTileCols) * cdiv(row_end - row_begin, amax_tile_h(kind, K, row_begin, row_end));
}

hipError_t launch_amax(int kind, const uint16_t* x, int64_t K, int64_t row_begin, int64_t row_end,
                       float* row_amax, float* col_amax, float* t0, float* t1, const GroupTable& gt,
                       hipStream_t st, const ZeroFirst& zero, const SyncArg& sync) {
    if (row_end <= row_begin || K <= 0) return hipSuccess;
    const int tile_h = amax_tile_h(kind, K, row_begin, row_end);
    dim3 grid(cdiv(K, kTileCols), cdiv(row_end - row_begin, tile_h));
    switch (kind) {
    case AMAX_TENSOR:
        hipLaunchKernelGGL(k_amax<AMAX_TENSOR>, grid, dim3(256), 0, st, x, K, row_begin, row_end, row_amax, col_amax, t0, t1, gt, tile_h, zero, sync);
        break;
    case AMAX_TOKEN:
        hipLaunchKernelGGL(k_amax<AMAX_TOKEN>, grid, dim3(256), 0, st, x, K, row_begin, row_end, row_amax, col_amax, t0, t1, gt, tile_h, zero, sync);
        break;
    default:
        hipLaunchKernelGGL(k_amax<AMAX_GROUPED>, grid, dim3(256), 0, st, x, K, row_begin, row_end, row_amax, col_amax, t0, t1, gt, tile_h, zero, sync);
        break;
    }
    return hipGetLastError();
}

// ev0 / ev1 (may be null): events the kernel's own dispatch records at its
// start and end, for timing it alone
template <int MODE, bool SAT, bool SWZ = false>
static void launch_encode_mode(bool row, bool col, dim3 grid, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1,
                               const uint16_t* x, int64_t M, int64_t K,
                               int64_t rb, int64_t re, const float* ra, const float* ca, uint8_t* rq, uint8_t* rs,
                               uint8_t* cq, uint8_t* cs, float* fr, float* fc, const GroupTable& gt, const Calib& cal,
                               int tile_h) {
    if (row && col)
        hipExtLaunchKernelGGL((k_encode<MODE, true, true, SAT, SWZ>), grid, dim3(256), 0, st, ev0, ev1, 0,
                              x, M, K, rb, re, ra, ca, rq, rs, cq, cs, fr, fc, gt, cal, tile_h);
    else if (row)
        hipExtLaunchKernelGGL((k_encode<MODE, true, false, SAT, SWZ>), grid, dim3(256), 0, st, ev0, ev1, 0,
                              x, M, K, rb, re, ra, ca, rq, rs, cq, cs, fr, fc, gt, cal, tile_h);
    else
        hipExtLaunchKernelGGL((k_encode<MODE, false, true, SAT, SWZ>), grid, dim3(256), 0, st, ev0, ev1, 0,
                              x, M, K, rb, re, ra, ca, rq, rs, cq, cs, fr, fc, gt, cal, tile_h);
}

hipError_t launch_encode(int mode, bool row, bool col, bool caller_amax, const uint16_t* x, int64_t M, int64_t K,
                         int64_t row_begin, int64_t row_end, const float* row_amax, const float* col_amax,
                         uint8_t* row_q, uint8_t* row_sf, uint8_t* col_q, uint8_t* col_sf,
                         float* fill_row, float* fill_col, const GroupTable& gt, hipStream_t st,
                         hipEvent_t ev0, hipEvent_t ev1, const Calib& cal, bool swizzled) {
    if (row_end <= row_begin || K <= 0 || (!row && !col)) return hipSuccess;
    // rows per workgroup: 256, or 128 when the grid would be small
    const int tile_h = (int64_t)cdiv(K, kEncCols) * cdiv(row_end - row_begin, kEncRows) < 768 ? 128 : kEncRows;
    dim3 grid(cdiv(K, kEncCols), cdiv(row_end - row_begin, tile_h));
#define NVFP4_ENC_ARGS row, col, grid, st, ev0, ev1, x, M, K, row_begin, row_end, row_amax, col_amax, row_q, row_sf, col_q, col_sf, fill_row, fill_col, gt, cal, tile_h
    if (swizzled) {
        // swizzled scales: per-tensor or per-token, amax computed here
        if (mode == ENC_TENSOR) launch_encode_mode<ENC_TENSOR, false, true>(NVFP4_ENC_ARGS);
        else launch_encode_mode<ENC_TOKEN, false, true>(NVFP4_ENC_ARGS);
    } else if (caller_amax) {
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

hipError_t launch_encode_sr(int mode, bool row, bool col, const uint16_t* x, int64_t M, int64_t K,
                            const float* row_amax, const float* col_amax, uint8_t* row_q, uint8_t* row_sf,
                            uint8_t* col_q, uint8_t* col_sf, uint64_t seed, uint32_t offset, hipStream_t st,
                            hipEvent_t ev0, hipEvent_t ev1) {
    if (M <= 0 || K <= 0 || (!row && !col)) return hipSuccess;
    const dim3 grid(cdiv(K, kEncCols), cdiv(M, 128));
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#define NVFP4_SR_LAUNCH(MD, R, C) hipExtLaunchKernelGGL((k_encode_sr<MD, R, C>), grid, dim3(256), 0, st, ev0, ev1, 0, \
                                                      x, M, K, row_amax, col_amax, row_q, row_sf, col_q, col_sf, k0, k1, offset)
    if (mode == ENC_TOKEN) {
        if (row && col) NVFP4_SR_LAUNCH(ENC_TOKEN, true, true);
        else if (row) NVFP4_SR_LAUNCH(ENC_TOKEN, true, false);
        else NVFP4_SR_LAUNCH(ENC_TOKEN, false, true);
    } else {
        if (row && col) NVFP4_SR_LAUNCH(ENC_TENSOR, true, true);
        else if (row) NVFP4_SR_LAUNCH(ENC_TENSOR, true, false);
        else NVFP4_SR_LAUNCH(ENC_TENSOR, false, true);
    }
#undef NVFP4_SR_LAUNCH
    return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* q, const uint8_t* sf, const float* amax, int64_t R, int64_t C,
                          int amax_per_row, bool bf16, void* out, hipStream_t st) {
    const int64_t blocks = R * (C / 16);
    if (blocks <= 0) return hipSuccess;
    unsigned grid = cdiv(blocks, 256);
    if (grid > 16384) grid = 16384;
    if (bf16) hipLaunchKernelGGL(k_dequant<true>, dim3(grid), dim3(256), 0, st, q, sf, amax, R, C, amax_per_row, out);
    else hipLaunchKernelGGL(k_dequant<false>, dim3(grid), dim3(256), 0, st, q, sf, amax, R, C, amax_per_row, out);
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
    hipLaunchKernelGGL(k_accumulate_reduce, dim3(1), dim3(1024), 0, st, buf, obs, n, decay);
    return hipGetLastError();
}

// ------------------------------------------------------- resident launcher

template <int MODE, bool ROW, bool COL>
static int resident_blocks_per_cu() {
    static int cached = -1;
    if (cached < 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(k_resident<MODE, ROW, COL>),
                                                         512, 0) != hipSuccess)
            n = 0;
        cached = n;
    }
    return cached;
}

int resident_blocks_per_cu(int mode, bool row, bool col) {
    if (mode == ENC_TOKEN) {
        if (row && col) return resident_blocks_per_cu<ENC_TOKEN, true, true>();
        if (row) return resident_blocks_per_cu<ENC_TOKEN, true, false>();
        return resident_blocks_per_cu<ENC_TOKEN, false, true>();
    }
    if (row && col) return resident_blocks_per_cu<ENC_TENSOR, true, true>();
    if (row) return resident_blocks_per_cu<ENC_TENSOR, true, false>();
    return resident_blocks_per_cu<ENC_TENSOR, false, true>();
}

hipError_t launch_resident(int mode, bool row, bool col, const ResArgs& a, unsigned grid, hipStream_t st,
                           hipEvent_t ev0, hipEvent_t ev1) {
    if (grid == 0 || (!row && !col)) return hipSuccess;
#define NVFP4_RES_LAUNCH(MD, R, C) hipExtLaunchKernelGGL((k_resident<MD, R, C>), dim3(grid), dim3(512), 0, st, ev0, ev1, 0, a)
    if (mode == ENC_TOKEN) {
        if (row && col) NVFP4_RES_LAUNCH(ENC_TOKEN, true, true);
        else if (row) NVFP4_RES_LAUNCH(ENC_TOKEN, true, false);
        else NVFP4_RES_LAUNCH(ENC_TOKEN, false, true);
    } else {
        if (row && col) NVFP4_RES_LAUNCH(ENC_TENSOR, true, true);
        else if (row) NVFP4_RES_LAUNCH(ENC_TENSOR, true, false);
        else NVFP4_RES_LAUNCH(ENC_TENSOR, false, true);
    }
#undef NVFP4_RES_LAUNCH
    return hipGetLastError();
}

}  // namespace nvfp4

// The Hadamard-transform cast, in this translation unit for its amax pass's
// cross-workgroup waits (the counters above).
#include "nvfp4_rht.inc"
