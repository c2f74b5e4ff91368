/*
 * nvfp4.h -- C ABI of libnvfp4: the bf16 -> NVFP4 block-scaled cast on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (TransformerEngine PR #3045, "Add NVFP4 per-token
 * quantization recipe": Description, Changes, and the sequence diagram of its
 * review summary):
 *   - an outer fp32 amax: one per tensor (the NVFP4BlockScaling default), or
 *     per token -- a vector of length M for rowwise output and a vector of
 *     length K for columnwise output;
 *   - per 16-element block, an FP8 E4M3 block scale relative to the outer
 *     scale S = amax / (6 * 448);
 *   - each element encoded to E2M1 and packed two per byte.
 * Exact arithmetic, for a vector v with outer amax A and block j:
 *   S = A/2688;  sf_j = (max|v in j| / 6) / S;  c_j = E4M3_rne_sat(sf_j);
 *   r_j = decode(c_j) * S;  nibble_i = E2M1_rne_sat(v_i / r_j)
 * with every step one IEEE binary32 operation rounded to nearest-even, and
 * S == 0 or r_j == 0 giving scale code 0 and sign-only nibbles.  The fp32
 * order of the block-scale formula follows the reading of the FP8 block-scale
 * discussion on Model-Optimizer PR #2598 (amax/6 relative to the global
 * scale); results are bit-identical to the library's CPU reference.
 *
 * Conventions shared by every entry point
 *   - x is bf16, contiguous row-major [M][K] (or [T][K] for grouped), on the
 *     device.  All other arrays are device memory owned by the caller; the
 *     library never reads outputs before writing them and allocates no
 *     device memory per call.  Its state: a thread-local error string and
 *     pending nvfp4_trace_encode pair, the nvfp4_set_schedule setting, and
 *     per device (set up at the first call there) the compute-unit count,
 *     the arrival counters of its cross-workgroup waits (a static device
 *     array) and one word of pinned host memory where a wait that gave up
 *     records it.
 *   - Rowwise output ("row_*"): row_q [M][K/2] bytes, row_sf [M][K/16] E4M3
 *     codes, row_amax fp32.  Columnwise output ("col_*") is the quantization
 *     of the transpose: col_q [K][M/2], col_sf [K][M/16], col_amax fp32.
 *     Element 2i sits in the low nibble of its byte; a nibble is
 *     sign<<3 | E2M1 magnitude code; scales are row-major and unswizzled.
 *   - amax lengths: per-tensor [1]; per-token rowwise [M], columnwise [K];
 *     16x16 tiles [M] and [K] filled with the tensor amax.
 *   - stream is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     work and return; results are ready when the stream reaches them.
 *   - Validation runs on the host before anything is enqueued.  On any
 *     non-OK status nothing was launched and nvfp4_last_error() names the
 *     problem.  NVFP4_EINVAL: NULL input, no direction requested, a NULL
 *     output in a requested direction, bad mode, decay outside [0,1],
 *     negative size.  NVFP4_ESHAPE: rowwise output needs K % 16 == 0,
 *     columnwise output M % 16 == 0 and K % 8 == 0, 16x16 tiles both
 *     M % 16 and K % 16; group counts must be >= 0 and % 16; every cast
 *     needs K < 2^25 (33554432) and M <= 2^40.
 *     NVFP4_EALIGN: a pointer not 16-byte aligned (amax/observed arrays need
 *     4-byte alignment).  NVFP4_EDEVICE: a HIP call or launch failed.
 *   - Outputs must not overlap the input or each other.  Inputs are assumed
 *     finite; a NaN or Inf input gives unspecified codes.
 *   - Any shape meeting these rules is accepted; all shapes give results
 *     bit-identical to the CPU reference.
 *   - The cast writes every amax output it computes: the arrays are zeroed
 *     on the stream (by the first workgroups of the launch that then
 *     max-combines into them, or by a launch before it), so their prior
 *     contents never matter.
 *   - Calls may be recorded by stream capture: on a capturing stream the
 *     library takes launch paths without cross-workgroup waits (whose
 *     arrival counts come from the host at each call).
 *   - Launches whose workgroups wait for one another bound every wait
 *     (about 0.2 s).  A wait that gives up -- possible only when other work
 *     holds the device's compute units for that long -- leaves that call's
 *     outputs invalid, and the next call on the device that launches such
 *     a kernel returns NVFP4_EDEVICE, once.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 3

#if defined(__GNUC__)
#define NVFP4_API __attribute__((visibility("default")))
#else
#define NVFP4_API
#endif

typedef enum {
    NVFP4_OK = 0,
    NVFP4_EINVAL = 1,
    NVFP4_ESHAPE = 2,
    NVFP4_EALIGN = 3,
    NVFP4_EDEVICE = 4
} nvfp4_status;

typedef enum {
    NVFP4_PER_TENSOR = 0,   /* one outer amax per tensor */
    NVFP4_PER_TOKEN = 1,    /* per-row amax (rowwise), per-column amax (columnwise) */
    NVFP4_TILE_16x16 = 2    /* one E4M3 scale per 16x16 tile, per-tensor amax */
} nvfp4_scaling;

NVFP4_API int nvfp4_abi_version(void);

/* Message for the last non-OK status returned on this thread ("" if none). */
NVFP4_API const char* nvfp4_last_error(void);

/*
 * Timing hook for benchmarks and profilers.  The next call on this thread
 * that launches the data-encoding kernel (the kernel that writes the packed
 * E2M1 bytes and the block scales) has that launch record `before` when the
 * kernel starts and `after` when it ends, so that hipEventElapsedTime gives
 * the kernel's own duration; the pair is then forgotten (one-shot).  A call
 * that fails validation leaves it pending; a grouped call times its first
 * encoding launch.  nvfp4_gemm and nvfp4_gemm_grouped take the pair the same
 * way for their GEMM kernel (a grouped GEMM over more than 128 groups runs
 * several launches: `before` at the first, `after` at the last).  Both
 * arguments are hipEvent_t handles created and owned
 * by the caller; NULL, NULL cancels a pending pair, and exactly one NULL is
 * NVFP4_EINVAL.  Recording the events changes no result.
 */
NVFP4_API nvfp4_status nvfp4_trace_encode(void* before, void* after);

/*
 * Launch schedule of the per-tensor and per-token casts whose amax the call
 * measures (nvfp4_quantize, _rowwise, _columnwise and _calibrate; the
 * swizzled, stochastic-rounding, Hadamard, grouped and 16x16 casts always
 * take the two-pass one):
 *   NVFP4_SCHEDULE_AUTO (default): resident where it applies and reads x
 *     once (at most two tiles per workgroup), else two-pass; per-token
 *     rowwise-only casts take their single-pass row kernel;
 *   NVFP4_SCHEDULE_TWO_PASS: an amax launch, then an encoding launch that
 *     reads x again;
 *   NVFP4_SCHEDULE_RESIDENT: the resident schedule wherever it applies,
 *     rowwise-only per-token casts included.
 * The resident schedule is one launch of at most one workgroup per compute
 * unit, all resident at once: an amax phase, a wait for every workgroup,
 * then an encoding phase, with the last two 256 x 256 tiles each workgroup
 * read in the amax phase encoded from registers (a tensor of at most two
 * such tiles per workgroup is read from memory once).  It applies when the
 * ceil(K/256) column strips fit that grid with runs of at most 32 tiles.
 * Every schedule gives bit-identical results; the setting exists for timing
 * comparisons and tests.  Process-wide, read at each call.  NVFP4_EINVAL for
 * another value.
 */
typedef enum {
    NVFP4_SCHEDULE_AUTO = 0,
    NVFP4_SCHEDULE_TWO_PASS = 1,
    NVFP4_SCHEDULE_RESIDENT = 2
} nvfp4_schedule;
NVFP4_API nvfp4_status nvfp4_set_schedule(nvfp4_schedule schedule);

/*
 * Testing hook for the failure path of the cross-workgroup waits: the next
 * launch on this process that waits on other workgroups gets an arrival
 * target no launch reaches, so each of its waits gives up at its bound
 * (about 0.2 s per waiting wave group, all in parallel) and the kernel
 * finishes without the work that depended on them.  That call returns
 * NVFP4_OK (its outputs are invalid); the next call on the device that
 * launches such a kernel returns NVFP4_EDEVICE once; calls after it are
 * normal.  Process-wide, one-shot; not for production use.
 */
NVFP4_API nvfp4_status nvfp4_test_fail_next_wait(void);

/*
 * Whole cast, one read of x serving both directions.  Pass NULL for all three
 * pointers of a direction that is not wanted (at least one must be wanted).
 * PER_TENSOR / PER_TOKEN follow the Description of the per-token recipe page;
 * TILE_16x16 is its opt-in 2D weight mode ("Changes": transposition-invariant
 * 16x16 cast emitted in per-token layout): one E4M3 code per tile relative to
 * the per-tensor outer scale, row_sf[m][J] = col_sf[k][I] = code of tile (I,J)
 * with I = m/16, J = k/16; nibbles identical in both directions.
 */
NVFP4_API nvfp4_status nvfp4_quantize(const void* x, int64_t M, int64_t K, nvfp4_scaling mode,
                            uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                            uint8_t* col_q, uint8_t* col_sf, float* col_amax,
                            void* stream);

/*
 * nvfp4_quantize followed by the decayed calibration update of the PTQ
 * scaling-factor page (TransformerEngine PR #3296, Description) on a scalar
 * buffer, in one call:  buf[0] = max(buf[0] * decay, A)  in fp32, where A is
 * the tensor amax this cast observed (the maximum of row_amax or col_amax
 * for PER_TOKEN, the tensor amax otherwise; 0 for an empty tensor).  The
 * result equals nvfp4_quantize then nvfp4_amax_accumulate_reduce on the
 * amax vector, without the second launch.  buf: one fp32 value in device
 * memory, finite and >= 0; decay in [0, 1].
 */
NVFP4_API nvfp4_status nvfp4_quantize_calibrate(const void* x, int64_t M, int64_t K, nvfp4_scaling mode,
                                      uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                                      uint8_t* col_q, uint8_t* col_sf, float* col_amax,
                                      float* buf, float decay, void* stream);

/*
 * nvfp4_quantize with stochastic rounding of the E2M1 element codes: the
 * stochastic-rounding variant the per-token recipe page lists next to the
 * per-token cast (TransformerEngine PR #3045, Changes), PER_TENSOR or
 * PER_TOKEN scaling (TILE_16x16 is NVFP4_EINVAL).  Outer amax and block scales
 * are those of nvfp4_quantize; each element's quotient x = |RN(v / r)| lies
 * in [lo, lo + d) of the E2M1 grid (d = 0.5 below 2, 1 below 4, 2 below 6)
 * and rounds up iff x - lo > U * d, U = R * 2^-8, R the element's 8-bit
 * random; x >= 6 saturates.  R is byte i % 16 of the Philox4x32-10 block
 * (Salmon et al., SC'11) with key (seed low word, seed high word) and
 * counter (i / 16, vector index, 0 for rowwise / 1 for columnwise, offset),
 * its four output words read as 16 little-endian bytes, where i is the
 * element's position along its vector (a row of x for rowwise output, a
 * column for columnwise output).  The page does not say
 * how its randoms are drawn; this is the library's definition, reproduced
 * bit for bit by its CPU reference.  The same seed and offset give the same
 * bytes; change offset per call for fresh randoms.  Needs M < 2^32
 * (NVFP4_ESHAPE otherwise).
 */
NVFP4_API nvfp4_status nvfp4_quantize_sr(const void* x, int64_t M, int64_t K, nvfp4_scaling mode,
                               uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                               uint8_t* col_q, uint8_t* col_sf, float* col_amax,
                               uint64_t seed, uint32_t offset, void* stream);

/*
 * Cast with the opt-in random Hadamard transform on the columnwise direction
 * (the per-token recipe page, PR #3045 "Changes": per_token_rht; the row
 * direction never uses it).  Rowwise outputs (optional: all three NULL to
 * skip) are exactly nvfp4_quantize's.  The columnwise outputs (required) are
 * nvfp4_quantize's columnwise cast of y instead of x, where each 16-element
 * block of a columnwise vector -- rows 16b .. 16b+15 of one column of x -- is
 *   y = H16 D x_block / 4
 * with H16 the Sylvester Hadamard matrix (H16[i][j] = (-1)^popcount(i & j))
 * and D = diag(s), s_i = -1 where bit i of sign_mask is set.  The pages fix
 * neither the size nor the arithmetic; this library evaluates y as the fast
 * Walsh-Hadamard butterfly in binary32 (stages 1, 2, 4, 8, each pair (a, b)
 * of entries i and i + h becoming (a + b, a - b)), multiplies by 1/4 and
 * rounds to bf16 nearest-even, then casts y with its own amax (col_amax: max
 * |y| per column for PER_TOKEN, over the tensor for PER_TENSOR).  Since H16 /
 * 4 is orthonormal and its own inverse, a consumer undoes the transform with
 * D H16 / 4 on the dequantized blocks.  mode PER_TENSOR or PER_TOKEN (else
 * EINVAL); sign_mask < 2^16 (EINVAL); M % 16 == 0 and K % 8 == 0 (plus K % 16
 * == 0 with rowwise output) and M <= 65535 * 128 (ESHAPE).  Reads x twice
 * in all (the amaxes of both directions, then both encodings).
 */
NVFP4_API nvfp4_status nvfp4_quantize_rht(const void* x, int64_t M, int64_t K, nvfp4_scaling mode,
                                uint32_t sign_mask,
                                uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                                uint8_t* col_q, uint8_t* col_sf, float* col_amax,
                                void* stream);

/* One direction only (same as nvfp4_quantize with the other direction NULL). */
NVFP4_API nvfp4_status nvfp4_quantize_rowwise(const void* x, int64_t M, int64_t K, nvfp4_scaling mode,
                                    uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                                    void* stream);
NVFP4_API nvfp4_status nvfp4_quantize_columnwise(const void* x, int64_t M, int64_t K, nvfp4_scaling mode,
                                       uint8_t* col_q, uint8_t* col_sf, float* col_amax,
                                       void* stream);

/*
 * Split form, first half: outer amax only ("K1 vector amax" on the per-token
 * page).  PER_TENSOR writes the tensor amax to whichever of row_amax /
 * col_amax is non-NULL ([1] each); PER_TOKEN writes row_amax [M] and/or
 * col_amax [K].  TILE_16x16 is not accepted here (it is PER_TENSOR's amax).
 */
NVFP4_API nvfp4_status nvfp4_amax(const void* x, int64_t M, int64_t K, nvfp4_scaling mode,
                        float* row_amax, float* col_amax, void* stream);

/*
 * Split form, second half ("K2 encode"): block scales and E2M1 data from
 * caller-supplied outer amax (e.g. calibrated values kept by
 * nvfp4_amax_accumulate).  PER_TENSOR reads row_amax[0] / col_amax[0];
 * PER_TOKEN reads row_amax [M] / col_amax [K].  An amax smaller than the
 * data's saturates: the block scale clamps to 448 (0x7E) and elements to 6.
 * A direction is requested by non-NULL q and sf (its amax must then be
 * non-NULL too).
 */
NVFP4_API nvfp4_status nvfp4_encode(const void* x, int64_t M, int64_t K, nvfp4_scaling mode,
                          const float* row_amax, const float* col_amax,
                          uint8_t* row_q, uint8_t* row_sf,
                          uint8_t* col_q, uint8_t* col_sf, void* stream);

/*
 * Grouped (MoE) per-token cast in one call: x holds T = sum(h_counts) rows of
 * K values, expert e owning rows [o_e, o_e + h_counts[e]) (the grouped
 * helper on the per-token page; zero-count experts are accepted -- they are
 * common under dynamic routing, as that page's review notes).
 *   rowwise  : per-token rowwise of all T rows: row_q [T][K/2], row_sf
 *              [T][K/16], row_amax [T];
 *   columnwise: per expert e, the columnwise quantization of its slice at
 *              byte offsets K*o_e/2 (col_q, [K][m_e/2]) and K*o_e/16
 *              (col_sf, [K][m_e/16]); col_amax is [num_groups][K] (a zero
 *              row for an empty expert).
 * h_counts is a HOST array of num_groups int64 values, each >= 0 and % 16.
 */
NVFP4_API nvfp4_status nvfp4_quantize_grouped(const void* x, int64_t K, int32_t num_groups,
                                    const int64_t* h_counts,
                                    uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                                    uint8_t* col_q, uint8_t* col_sf, float* col_amax,
                                    void* stream);

/*
 * Dequantize R vectors of C values (C % 16 == 0, else ESHAPE) from q [R][C/2]
 * and sf [R][C/16] to out [R][C]: this is the reference dequantization the
 * per-token page pairs with its quantizer (TransformerEngine PR #3045,
 * Important Files Changed: the per-token GEMM test's reference dequant).
 *   out = (+/-) g * (decode(sf) * (A / 2688)),
 * the product computed exactly as in the cast (one binary32 multiply by the
 * same divisor r), with A = amax[r] for mode NVFP4_PER_TOKEN (amax holds R
 * values) and A = amax[0] for NVFP4_PER_TENSOR and NVFP4_TILE_16x16 (a 16x16
 * cast already replicates each tile's scale byte per vector and fills its
 * amax vectors with the tensor amax); another mode is EINVAL.
 * out_is_bf16 == 0: out is fp32; otherwise out is bf16, each value the
 * round-to-nearest-even (ties to even) of that fp32 value.  Columnwise
 * buffers are passed with R = K, C = M.  q 8-byte, out 16-byte and amax
 * 4-byte aligned (EALIGN); NULL pointers with R, C > 0 are EINVAL; R == 0 or
 * C == 0 does nothing.  The caller owns every buffer; nothing is allocated.
 */
NVFP4_API nvfp4_status nvfp4_dequantize(const uint8_t* q, const uint8_t* sf, const float* amax,
                              int64_t R, int64_t C, nvfp4_scaling mode, int out_is_bf16, void* out,
                              void* stream);

/*
 * NVFP4 GEMM consumer: the GEMM of the per-token recipe page (TransformerEngine
 * PR #3045, Changes and the sequence diagram's TN forward product) that
 * rescales with the per-row / per-column outer amax vectors in its epilogue.
 * A and B are NVFP4 with 16-element blocks along K: a_q [M][K/2], a_sf
 * [M][K/16], a_amax [M] (a_per_row != 0) or [1]; likewise b_* with N rows.
 *   out[m][n] = S_a(m) * S_b(n) * sum_k (g * D)_a[m][k] * (g * D)_b[n][k]
 * with g the E2M1 value, D the decoded block scale, S = amax / 2688 (as in the
 * cast), out fp32 row-major [M][N], written in full (zeros when K == 0).  The
 * page's forward (TN: x rowwise, W rowwise), dgrad (NN: dY rowwise, W
 * columnwise) and wgrad (NT: dY columnwise, x columnwise) products are this
 * call on the cast's outputs.  The sum runs in fp32 on fp16 matrix cores (the
 * block values g * D are exact in fp16); against the exact value the error is
 * within (K + 2) * 2^-24 * S_a * S_b * sum_k |term|.  K % 16 == 0 (ESHAPE);
 * K <= 2^23 (ESHAPE); a_q, b_q 16-byte aligned, amax and out 4-byte aligned
 * (EALIGN); at most 2^31 - 1 output tiles of 128 x 128, cdiv(M, 128) *
 * cdiv(N, 128) (ESHAPE).
 * M == 0 or N == 0 does nothing; negative sizes or NULL pointers (the
 * operands may be NULL only when K == 0) give EINVAL.  Nothing is allocated.
 */
NVFP4_API nvfp4_status nvfp4_gemm(const uint8_t* a_q, const uint8_t* a_sf, const float* a_amax, int a_per_row,
                        const uint8_t* b_q, const uint8_t* b_sf, const float* b_amax, int b_per_row,
                        int64_t M, int64_t N, int64_t K, float* out, void* stream);

/*
 * GEMM-swizzled scale layout.  The per-token recipe page emits unswizzled
 * scales and leaves the swizzled layout to its GEMM (PR #3045: GEMM-swizzled
 * scales off, with_swizzle=0) without defining it; this library takes the
 * tiled layout of block-scaled GEMMs for 16-element FP4 blocks.  For a plain
 * scale matrix sf [R][nb] (row r, block c; nb = C/16), with Rp = R rounded
 * up to 128 and nbp = nb rounded up to 4, the swizzled buffer holds Rp * nbp
 * bytes in 512-byte tiles of 128 rows x 4 blocks, row-tile major:
 *   byte(r, c) = 512 * ((r / 128) * (nbp / 4) + c / 4)
 *              + 16 * (r % 32) + 4 * ((r / 32) % 4) + c % 4
 * and every byte no (r < R, c < nb) maps to is zero.  A row's four blocks of
 * a tile sit in one 4-byte word.
 *
 * nvfp4_swizzle_scales writes all Rp * nbp bytes of `out` (4-byte aligned,
 * EALIGN) from plain sf [R][nb] (e.g. the cast's row_sf with nb = K/16, or
 * col_sf with R = K, nb = M/16).  Sizes < 0: EINVAL.
 */
NVFP4_API nvfp4_status nvfp4_swizzle_scales(const uint8_t* sf, int64_t R, int64_t nb, uint8_t* out,
                                  void* stream);

/*
 * nvfp4_quantize with both scale outputs written directly in the swizzled
 * layout above: row_sf as the [M][K/16] matrix, col_sf as [K][M/16], each
 * M*K/16 bytes (no padding: M % 128 == 0 and K % 128 == 0, else ESHAPE; M*K/16
 * < 2^31).  Every other output byte equals nvfp4_quantize's, and the scales
 * equal nvfp4_swizzle_scales of its scales.  PER_TENSOR or PER_TOKEN (else
 * EINVAL); row_sf and col_sf 4-byte aligned (EALIGN).  Each workgroup of the
 * encoding kernel writes whole 512-byte tiles of both scale matrices.
 */
NVFP4_API nvfp4_status nvfp4_quantize_swizzled(const void* x, int64_t M, int64_t K, nvfp4_scaling mode,
                                     uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                                     uint8_t* col_q, uint8_t* col_sf, float* col_amax,
                                     void* stream);

/*
 * nvfp4_gemm with both operands' scales in the swizzled layout above (a_sf
 * of R = M rows, b_sf of R = N rows, nb = K/16 each; 4-byte aligned, EALIGN).
 * Same arithmetic, results bit-identical to nvfp4_gemm on the plain scales.
 */
NVFP4_API nvfp4_status nvfp4_gemm_swizzled(const uint8_t* a_q, const uint8_t* a_sf, const float* a_amax,
                                 int a_per_row, const uint8_t* b_q, const uint8_t* b_sf,
                                 const float* b_amax, int b_per_row, int64_t M, int64_t N, int64_t K,
                                 float* out, void* stream);

/*
 * Grouped NVFP4 GEMM for MoE experts, one launch per 128 groups (the page's
 * native grouped per-token GEMM over a pointer array of experts, PR #3045
 * "Changes"): A holds the tokens of num_groups experts back to back, h_counts
 * (a HOST array of num_groups values >= 0, any size) rows each -- the
 * rowwise output of nvfp4_quantize_grouped has this layout -- with a_q
 * [T][K/2], a_sf [T][K/16], a_amax [T] (a_per_row != 0) or [1].  Expert e's
 * weight B_e is b_q + e*N*K/2 ([N][K/2]), b_sf + e*N*K/16, b_amax + e*N
 * ([G][N], b_per_row != 0) or b_amax + e ([G], one per expert).  The rows
 * of expert e in out [T][N] fp32 get A_e x B_e^T with the outer scales, each
 * element exactly as nvfp4_gemm computes it.  Same limits and errors as
 * nvfp4_gemm, plus EINVAL for num_groups < 0 or a NULL h_counts, and ESHAPE
 * for a negative count.
 */
NVFP4_API nvfp4_status nvfp4_gemm_grouped(const uint8_t* a_q, const uint8_t* a_sf, const float* a_amax,
                                int a_per_row, const uint8_t* b_q, const uint8_t* b_sf,
                                const float* b_amax, int b_per_row, int32_t num_groups,
                                const int64_t* h_counts, int64_t N, int64_t K, float* out,
                                void* stream);

/*
 * Decayed calibration accumulator from the PTQ scaling-factor page
 * (TransformerEngine PR #3296, Description): buf[i] = max(buf[i] * decay,
 * observed[i]) for i < n, in fp32.  decay 0 keeps the latest value, decay 1
 * the maximum over the whole history.  decay must lie in [0, 1].
 */
NVFP4_API nvfp4_status nvfp4_amax_accumulate(float* buf, const float* observed, int64_t n, float decay,
                                   void* stream);

/*
 * Scalar form for per-token recipes: the same page max-reduces the row-wise
 * vector to a scalar, so buf[0] = max(buf[0] * decay, max_i observed[i]) (an
 * empty vector observes 0).
 */
NVFP4_API nvfp4_status nvfp4_amax_accumulate_reduce(float* buf, const float* observed, int64_t n,
                                          float decay, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_H */
