// nvfp4_internal.h -- launchers shared between the C ABI (nvfp4_api.cpp) and
// the kernel translation units.  Not part of the public interface.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

struct GroupTable;

enum AmaxKind { AMAX_TENSOR = 0, AMAX_TOKEN = 1, AMAX_GROUPED = 2 };

// Cross-workgroup waits (nvfp4_kernels.hip): a launch that needs them gets a
// slot of monotonically increasing arrival counters in device memory, the
// slot's count when it starts (base), and a word of host memory (seen by the
// device) where a wait that gave up records the failure.  The host hands
// out slots in turn and advances each slot's base by the launch's
// arrivals, so a slot is shared only by launches kSyncSlots calls apart.
constexpr int kSyncSlots = 64;
struct SyncArg {
    unsigned long long base;
    unsigned int* err;
    int slot;   // -1: the launch needs no waits
};
enum EncodeMode { ENC_TENSOR = 0, ENC_TOKEN = 1, ENC_TILE = 2, ENC_GROUPED = 3 };

// the encoding kernel forms 32-bit byte offsets within 32 rows of x
constexpr int64_t kMaxEncodeK = int64_t(1) << 25;

hipError_t launch_fill2(float* p, int64_t n, float* q, int64_t m, float v, hipStream_t st);
// zero (with sync.slot >= 0): the first `wgs` workgroups (in dispatch
// order) zero a[0..na) and b[0..nb) between them, kZeroPerWg values each,
// and arrive; every workgroup waits for those `wgs` arrivals before
// combining into the outputs.  Without it the outputs must already hold
// zeros.
constexpr int64_t kZeroPerWg = 16384;
struct ZeroFirst {
    float* a;
    int64_t na;
    float* b;
    int64_t nb;
    int wgs;
};
// workgroups of the amax launch for these rows (0 when there is nothing to do)
int64_t amax_grid_size(int kind, int64_t K, int64_t row_begin, int64_t row_end);
hipError_t launch_amax(int kind, const uint16_t* x, int64_t K, int64_t row_begin, int64_t row_end,
                       float* row_amax, float* col_amax, float* t0, float* t1, const GroupTable& gt,
                       hipStream_t st, const ZeroFirst& zero = ZeroFirst{nullptr, 0, nullptr, 0, 0},
                       const SyncArg& sync = SyncArg{0ull, nullptr, -1});
// optional calibration update done by the encoding kernel: buf[0] =
// max(buf[0] * decay, max(obs[0..n))); buf == nullptr: none
struct Calib {
    float* buf;
    const float* obs;
    int64_t n;
    float decay;
};

// Resident one-launch cast (per-tensor or per-token, amax measured in the
// same launch; nvfp4_kernels.hip): 256 x 256 tiles, workgroup w takes a
// vertical run of up to `run` tiles of strip w / nband, band w % nband; the
// grid (ceil(K / 256) * nband workgroups of 512 lanes) must be resident at
// once.  zero / zsync: zero-first of the amax outputs (zsync.slot < 0: they
// hold zeros already); bar: the grid-wide wait.
struct ResArgs {
    const uint16_t* x;
    int64_t M, K;
    float* row_amax;
    float* col_amax;
    uint8_t* row_q;
    uint8_t* row_sf;
    uint8_t* col_q;
    uint8_t* col_sf;
    int run, nband;
    ZeroFirst zero;
    SyncArg zsync, bar;
    Calib cal;
};
// workgroups of the resident kernel one compute unit holds (0 when unknown)
int resident_blocks_per_cu(int mode, bool row, bool col);
hipError_t launch_resident(int mode, bool row, bool col, const ResArgs& a, unsigned grid, hipStream_t st,
                           hipEvent_t ev0, hipEvent_t ev1);

hipError_t launch_encode(int mode, bool row, bool col, bool caller_amax, const uint16_t* x, int64_t M, int64_t K,
                         int64_t row_begin, int64_t row_end, const float* row_amax, const float* col_amax,
                         uint8_t* row_q, uint8_t* row_sf, uint8_t* col_q, uint8_t* col_sf,
                         float* fill_row, float* fill_col, const GroupTable& gt, hipStream_t st,
                         hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr, const Calib& cal = Calib{nullptr, nullptr, 0, 0.0f},
                         bool swizzled = false);   // swizzled: mode ENC_TENSOR/ENC_TOKEN, M and K % 128 == 0
// stochastic-rounding cast (mode ENC_TENSOR or ENC_TOKEN; amax computed before)
hipError_t launch_encode_sr(int mode, bool row, bool col, const uint16_t* x, int64_t M, int64_t K,
                            const float* row_amax, const float* col_amax, uint8_t* row_q, uint8_t* row_sf,
                            uint8_t* col_q, uint8_t* col_sf, uint64_t seed, uint32_t offset, hipStream_t st,
                            hipEvent_t ev0, hipEvent_t ev1);
// random Hadamard transform + columnwise cast, with the ordinary rowwise cast
// of x when row_q != nullptr (nvfp4_rht.inc): amax outputs ([K] / [M] per
// token, [1] per tensor) zeroed beforehand, or by the amax launch's first
// workgroups (zero, sync as for launch_amax); M % 16 == 0, K % 8 == 0 (K %
// 16 == 0 with rows)
hipError_t launch_rht(int mode, const uint16_t* x, int64_t M, int64_t K, uint32_t mask, float* row_amax,
                      float* col_amax, uint8_t* row_q, uint8_t* row_sf, uint8_t* col_q, uint8_t* col_sf, hipStream_t st,
                      hipEvent_t ev0, hipEvent_t ev1, const ZeroFirst& zero = ZeroFirst{nullptr, 0, nullptr, 0, 0},
                      const SyncArg& sync = SyncArg{0ull, nullptr, -1}, bool* amax_launched = nullptr);
// workgroups of the Hadamard amax launch
int64_t rht_amax_grid_size(int64_t M, int64_t K);
// NVFP4 GEMM consumer (nvfp4_gemm.hip): out [M][N] fp32, one workgroup per
// 128 x 128 output tile, at most kMaxGemmTiles of them
constexpr int64_t kMaxGemmTiles = (int64_t(1) << 31) - 1;
// the GEMM kernel addresses a tile's operand rows with 32-bit byte offsets
constexpr int64_t kMaxGemmK = int64_t(1) << 23;
// swizzled: both operands' scales in the GEMM-swizzled layout
hipError_t launch_gemm_nvfp4(const uint8_t* a_q, const uint8_t* a_sf, const float* a_amax, int a_per_row,
                             const uint8_t* b_q, const uint8_t* b_sf, const float* b_amax, int b_per_row,
                             int64_t M, int64_t N, int64_t K, float* out, hipStream_t st, hipEvent_t ev0,
                             hipEvent_t ev1, bool swizzled);
// plain scales [R][nb] -> GEMM-swizzled layout (out 4-byte aligned, all of
// its ceil(R/128)*128 * ceil(nb/4)*4 bytes written)
hipError_t launch_swizzle_scales(const uint8_t* sf, int64_t R, int64_t nb, uint8_t* out, hipStream_t st);
// grouped GEMM: groups of A's rows, each with its own B, a bounded number per
// launch (the table travels in the kernel arguments)
constexpr int kMaxGemmGroups = 128;
struct GemmGroups {
    int32_t n;                              // entries in this launch
    int32_t first;                          // expert index of entry 0
    int64_t off[kMaxGemmGroups];            // first row of A / out
    int64_t cnt[kMaxGemmGroups];            // rows
    uint32_t tstart[kMaxGemmGroups + 1];    // first output tile of each entry; tstart[n]: all tiles
};
hipError_t launch_gemm_grouped(const uint8_t* a_q, const uint8_t* a_sf, const float* a_amax, int a_per_row,
                               const uint8_t* b_q, const uint8_t* b_sf, const float* b_amax, int b_per_row,
                               int32_t num_groups, const int64_t* h_counts, int64_t N, int64_t K, float* out,
                               hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);
// out: fp32 [R][C], or bf16 (round to nearest-even of the fp32 value) when bf16
hipError_t launch_dequant(const uint8_t* q, const uint8_t* sf, const float* amax, int64_t R, int64_t C,
                          int amax_per_row, bool bf16, void* out, hipStream_t st);
// single-pass per-token rowwise cast (nvfp4_rows.hip): rounds of 4096
// columns per row for K (1, 2, 4, 8 or 16), 0 when K is beyond the kernel
int rows_rounds(int64_t K);
// batches of rows for M x K (grid sizes are at most this)
int64_t rows_batches(int64_t M, int64_t K);
// row_q / row_sf / row_amax written in full
hipError_t launch_rows(const uint16_t* x, int64_t M, int64_t K, uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                       unsigned grid, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_accumulate(float* buf, const float* obs, int64_t n, float decay, hipStream_t st);
hipError_t launch_accumulate_reduce(float* buf, const float* obs, int64_t n, float decay, hipStream_t st);

}  // namespace nvfp4
