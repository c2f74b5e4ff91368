/*
 * nvfp4_oracle.h -- plain, slow CPU reference for the bf16 -> NVFP4
 * block-scaled cast.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check
 * and the benchmark's CPU-baseline leg may call it; the product library never
 * does, and this header shares nothing with the library's own header.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] TransformerEngine PR #3296 "[PTQ] Store FP32 global scaling factors
 *        (absmax or scale_inv) for all quantized activations and weights",
 *        section "Description" (decayed max accumulator, max-reduce of the
 *        row-wise vector to a scalar).
 *   [P2] TransformerEngine PR #3045 "Add NVFP4 per-token quantization
 *        recipe", sections "Description", "Changes", the Greptile summary
 *        and its sequence diagram (per-row / per-col outer amax, K1 vector
 *        amax + K2 encode, 2D 16x16 weight mode, grouped helper).
 *   [P5] Model-Optimizer PR #2598 (fused GPTQ update by default), review
 *        thread on how the FP8 block scale is formed from amax/6 and 448.
 *
 * Every floating-point step is one IEEE-754 binary32 operation with
 * round-to-nearest-even; the file is compiled with -ffp-contract=off so no
 * multiply-add is fused.  All buffers are host memory owned by the caller.
 * x is bf16 bit patterns (uint16), row-major with leading dimension ld.
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* scalar codecs */
float   orc_bf16_to_f32(uint16_t b);
uint8_t orc_e4m3_encode(float s);      /* s >= 0: RNE onto OCP E4M3, saturates at 448 */
float   orc_e4m3_decode(uint8_t code);
uint8_t orc_e2m1_encode(float q);      /* RNE onto {0,.5,1,1.5,2,3,4,6}, saturating, sign copied */
float   orc_e2m1_decode(uint8_t nibble);

/* array forms of the codecs (for the pin tests) */
void orc_e4m3_encode_array(const float* s, int64_t n, uint8_t* out);
void orc_e2m1_encode_array(const float* q, int64_t n, uint8_t* out);

/* core routine: one vector of n values (n % 16 == 0) with outer amax A.
 * q receives n/2 packed bytes (element 2i in the low nibble), sf n/16 E4M3
 * codes. */
void orc_quantize_vector(const float* v, int64_t n, float A, uint8_t* q, uint8_t* sf);

/* outer amax */
float orc_amax_tensor(const uint16_t* x, int64_t M, int64_t K, int64_t ld);
void  orc_amax_rows(const uint16_t* x, int64_t M, int64_t K, int64_t ld, float* out);
void  orc_amax_cols(const uint16_t* x, int64_t M, int64_t K, int64_t ld, float* out);

/* encode with caller-supplied outer amax.  per_vector = 0: amax[0] for all
 * vectors; 1: one amax per row (rowwise) or per column (columnwise).
 * rowwise : q [M][K/2],  sf [M][K/16]
 * colwise : q [K][M/2],  sf [K][M/16]  (quantization of the transpose) */
int orc_encode_rowwise(const uint16_t* x, int64_t M, int64_t K, int64_t ld,
                       int per_vector, const float* amax, uint8_t* q, uint8_t* sf);
int orc_encode_colwise(const uint16_t* x, int64_t M, int64_t K, int64_t ld,
                       int per_vector, const float* amax, uint8_t* q, uint8_t* sf);

/* whole cast.  mode 0 = per-tensor, 1 = per-token, 2 = 16x16 tiles.
 * Any of the row_* / col_* groups may be NULL (direction not requested).
 * amax outputs: mode 0 -> [1]; mode 1 -> [M] and [K]; mode 2 -> [M] and [K]
 * filled with the tensor amax.  Returns 0, or -1 on a shape error. */
int orc_quantize(const uint16_t* x, int64_t M, int64_t K, int mode,
                 uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                 uint8_t* col_q, uint8_t* col_sf, float* col_amax);

/* grouped per-token cast over G experts with row counts counts[e].
 * rowwise: per-token rowwise of the concatenation (row_amax [sum]);
 * colwise: expert e at byte offsets K*o_e/2 (data) and K*o_e/16 (scales),
 * each [K][m_e/2] and [K][m_e/16]; col_amax [G][K]. */
int orc_quantize_grouped(const uint16_t* x, int64_t K, int32_t G, const int64_t* counts,
                         uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                         uint8_t* col_q, uint8_t* col_sf, float* col_amax);

/* dequantize R vectors of C values: out[r][c] = (+/-) g * (D * (A/2688)).
 * amax_per_row = 0: amax[0] for all rows; 1: amax[r]. */
int orc_dequantize(const uint8_t* q, const uint8_t* sf, const float* amax,
                   int64_t R, int64_t C, int amax_per_row, float* out);

/* decayed accumulator: buf[i] = max(buf[i] * decay, obs[i]) */
void orc_amax_accumulate(float* buf, const float* obs, int64_t n, float decay);
/* scalar form fed by the max of a vector: buf[0] = max(buf[0]*decay, max_i obs[i]) */
void orc_amax_accumulate_reduce(float* buf, const float* obs, int64_t n, float decay);


/* stochastic-rounding variant (definition and readings in nvfp4_oracle.c) */
void    orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
void    orc_philox4x32_10_array(const uint32_t* ctr, const uint32_t* key, int64_t n, uint32_t* out);
uint8_t orc_e2m1_encode_sr(float q, uint8_t rnd);
void    orc_e2m1_encode_sr_array(const float* q, const uint8_t* rnd, int64_t n, uint8_t* out);
void    orc_quantize_vector_sr(const float* v, int64_t n, float A, uint8_t* q, uint8_t* sf,
                               uint64_t seed, uint32_t vec, uint32_t dir, uint32_t offset);
int     orc_quantize_sr(const uint16_t* x, int64_t M, int64_t K, int mode,
                        uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                        uint8_t* col_q, uint8_t* col_sf, float* col_amax,
                        uint64_t seed, uint32_t offset);


/* GEMM consumer: out[m][n] = S_a(m) S_b(n) sum_k (gD)_a[m][k] (gD)_b[n][k] in
 * binary64 (definition in nvfp4_oracle.c); bound may be NULL */
int orc_gemm_nvfp4(const uint8_t* aq, const uint8_t* asf, const float* aamax, int a_per_row,
                   const uint8_t* bq, const uint8_t* bsf, const float* bamax, int b_per_row,
                   int64_t M, int64_t N, int64_t K, double* out, double* bound);

/* random Hadamard transform of 16 bf16 values (binary32 butterfly, 1/4,
 * bf16 result; definition and readings in nvfp4_oracle.c), and of every
 * 16-row block down the columns of x [M][K] */
void orc_rht16(const uint16_t in[16], uint32_t sign_mask, uint16_t out[16]);
int  orc_rht_columns(const uint16_t* x, int64_t M, int64_t K, uint32_t sign_mask, uint16_t* y);

/* GEMM-swizzled scale layout (definition in nvfp4_oracle.c): size in bytes,
 * plain [R][nb] -> swizzled (padding zeroed) and back */
int64_t orc_swizzled_size(int64_t R, int64_t nb);
int     orc_swizzle_scales(const uint8_t* sf, int64_t R, int64_t nb, uint8_t* out);
int     orc_unswizzle_scales(const uint8_t* in, int64_t R, int64_t nb, uint8_t* sf);

#ifdef __cplusplus
}
#endif
/* Per-token row + column cast with rows and columns partitioned over
 * nthreads threads (1 .. 1024), each running the per-vector routines above
 * on its share; for timing the oracle on the host's cores.  Returns 0, or
 * -1 on bad arguments. */
int orc_quantize_per_token_threads(const uint16_t* x, int64_t M, int64_t K, int nthreads,
                                   uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                                   uint8_t* col_q, uint8_t* col_sf, float* col_amax);

#endif
