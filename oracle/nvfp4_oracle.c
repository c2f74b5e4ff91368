/*
 * nvfp4_oracle.c -- plain, slow CPU reference for the bf16 -> NVFP4
 * block-scaled cast.  TEST INFRASTRUCTURE ONLY (tests, smoke check, the
 * benchmark's CPU-baseline leg).  It shares no code with the HIP library.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math (oracle/build.py).
 *
 * What is computed, for one vector v of n values (n % 16 == 0) with outer
 * amax A (the steps follow the per-token recipe page, TransformerEngine
 * PR #3045, "Description"/"Changes" and the sequence diagram, and the block
 * scale discussion on Model-Optimizer PR #2598):
 *   S    = A / 2688                (2688 = 6 * 448: E2M1 max times E4M3 max)
 *   b_j  = max |v| over block j of 16 values
 *   sf_j = (b_j / 6) / S           two divisions, in this order
 *   c_j  = E4M3(sf_j), D_j = decode(c_j)
 *   r_j  = D_j * S
 *   nib  = E2M1(v_i / r_j)         division, then RNE onto the E2M1 grid
 * with S == 0 or r_j == 0 giving scale code 0 and sign-only nibbles.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - block-scale op order (b/6)/S: the Model-Optimizer review shows two
 *     orders disagree on ~0.1% of blocks; this one is fixed by convention
 *     (parity of that choice is unpinned by the pages).
 *   - sign of zero copied into the nibble; even element in the low nibble;
 *     zero outer amax or zero block scale gives code 0 and sign-only
 *     nibbles (conventions, unpinned).
 */
#include "nvfp4_oracle.h"

#include <math.h>
#include <string.h>
#include <pthread.h>
#include <stdlib.h>

/* ---------------------------------------------------------------- codecs */

float orc_bf16_to_f32(uint16_t b)
{
    /* bf16 is the high half of a binary32: widening is exact */
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* round a non-negative float that holds an exact value to the nearest
 * integer, ties to even (written out rather than relying on the FP
 * environment's rounding mode) */
static float round_half_even(float y)
{
    float fl = floorf(y);
    float frac = y - fl;            /* exact: y and fl share the binade scale */
    if (frac > 0.5f) return fl + 1.0f;
    if (frac < 0.5f) return fl;
    /* tie: pick the even neighbour */
    return (fmodf(fl, 2.0f) == 0.0f) ? fl : fl + 1.0f;
}

/* OCP FP8 E4M3 ("fn"): bias 7, 3 mantissa bits, no infinities, 0x7F is NaN,
 * largest finite value 448 (0x7E), subnormals m * 2^-9. */
float orc_e4m3_decode(uint8_t code)
{
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    float mag;
    if (e == 0)
        mag = ldexpf((float)m, -9);
    else
        mag = ldexpf((float)(8 + m), e - 10);   /* (1 + m/8) * 2^(e-7) */
    if (e == 0xF && m == 0x7) mag = NAN;
    return (code & 0x80) ? -mag : mag;
}

uint8_t orc_e4m3_encode(float s)
{
    /* s >= 0 by construction (a ratio of magnitudes).  Values at or above the
     * largest finite code saturate to it; (448, 464] would round there anyway. */
    if (!(s < 448.0f)) return 0x7E;
    if (s <= 0.0f) return 0x00;
    if (s < ldexpf(1.0f, -6)) {
        /* subnormal range: quantum 2^-9, code == integer multiple */
        float m = round_half_even(ldexpf(s, 9));  /* exact scaling by 2^9 */
        return (uint8_t)m;                         /* m == 8 is code 0x08 = 2^-6 */
    }
    int fe;
    (void)frexpf(s, &fe);          /* s = f * 2^fe, f in [0.5, 1) */
    int e = fe - 1;                /* floor(log2 s), in [-6, 8] here */
    float m = round_half_even(ldexpf(s, 3 - e));   /* significand * 8, in [8, 16] */
    if (m >= 16.0f) { m = 8.0f; e += 1; }
    int code = ((e + 7) << 3) | ((int)m - 8);
    if (code > 0x7E) code = 0x7E;
    return (uint8_t)code;
}

/* E2M1 magnitudes, code 0..7 */
static const float kE2M1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

float orc_e2m1_decode(uint8_t nibble)
{
    float g = kE2M1[nibble & 7];
    return (nibble & 8) ? -g : g;
}

uint8_t orc_e2m1_encode(float q)
{
    /* round to nearest, ties to the even code, saturating at 6; the
     * comparison list is the grid's midpoints with the tie direction of each */
    uint8_t s = signbit(q) ? 8 : 0;
    float a = fabsf(q);
    uint8_t c;
    if (a <= 0.25f)      c = 0;   /* tie 0.25 -> 0 (even) */
    else if (a < 0.75f)  c = 1;   /* tie 0.75 -> 1.0 (code 2) */
    else if (a <= 1.25f) c = 2;   /* tie 1.25 -> 1.0 */
    else if (a < 1.75f)  c = 3;   /* tie 1.75 -> 2.0 (code 4) */
    else if (a <= 2.5f)  c = 4;   /* tie 2.5  -> 2.0 */
    else if (a < 3.5f)   c = 5;   /* tie 3.5  -> 4.0 (code 6) */
    else if (a <= 5.0f)  c = 6;   /* tie 5.0  -> 4.0 */
    else                 c = 7;   /* beyond: saturate at 6 (also +inf) */
    return (uint8_t)(s | c);
}

void orc_e4m3_encode_array(const float* s, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(s[i]);
}

void orc_e2m1_encode_array(const float* q, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_encode(q[i]);
}

/* ------------------------------------------------------------ core routine */

static const float kE2M1Max = 6.0f;
static const float kOuterDiv = 2688.0f;   /* 6 * 448, exact */

/* quantize the 16 values of one block given its decoded ratio r = D * S */
static void encode_block(const float* v, int64_t count, float r, uint8_t* nibbles)
{
    for (int64_t i = 0; i < count; ++i) {
        if (r == 0.0f)
            nibbles[i] = signbit(v[i]) ? 8 : 0;
        else
            nibbles[i] = orc_e2m1_encode(v[i] / r);
    }
}

void orc_quantize_vector(const float* v, int64_t n, float A, uint8_t* q, uint8_t* sf)
{
    float S = A / kOuterDiv;
    uint8_t nib[16];
    for (int64_t j = 0; j < n / 16; ++j) {
        const float* blk = v + 16 * j;
        float r;
        if (S == 0.0f) {
            sf[j] = 0x00;
            r = 0.0f;
        } else {
            float b = 0.0f;
            for (int i = 0; i < 16; ++i) {
                float a = fabsf(blk[i]);
                if (a > b) b = a;
            }
            float t = b / kE2M1Max;
            float s = t / S;
            uint8_t code = orc_e4m3_encode(s);
            sf[j] = code;
            r = orc_e4m3_decode(code) * S;
        }
        encode_block(blk, 16, r, nib);
        for (int i = 0; i < 8; ++i)
            q[8 * j + i] = (uint8_t)(nib[2 * i] | (nib[2 * i + 1] << 4));
    }
}

/* ------------------------------------------------------------------ amax */

float orc_amax_tensor(const uint16_t* x, int64_t M, int64_t K, int64_t ld)
{
    float A = 0.0f;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(orc_bf16_to_f32(x[m * ld + k]));
            if (a > A) A = a;
        }
    return A;
}

void orc_amax_rows(const uint16_t* x, int64_t M, int64_t K, int64_t ld, float* out)
{
    for (int64_t m = 0; m < M; ++m) {
        float A = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(orc_bf16_to_f32(x[m * ld + k]));
            if (a > A) A = a;
        }
        out[m] = A;
    }
}

void orc_amax_cols(const uint16_t* x, int64_t M, int64_t K, int64_t ld, float* out)
{
    for (int64_t k = 0; k < K; ++k) {
        float A = 0.0f;
        for (int64_t m = 0; m < M; ++m) {
            float a = fabsf(orc_bf16_to_f32(x[m * ld + k]));
            if (a > A) A = a;
        }
        out[k] = A;
    }
}

/* ---------------------------------------------------------------- modes */

int orc_encode_rowwise(const uint16_t* x, int64_t M, int64_t K, int64_t ld,
                       int per_vector, const float* amax, uint8_t* q, uint8_t* sf)
{
    if (M < 0 || K < 0 || K % 16 != 0) return -1;
    float* v = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k) v[k] = orc_bf16_to_f32(x[m * ld + k]);
        float A = per_vector ? amax[m] : amax[0];
        orc_quantize_vector(v, K, A, q + m * (K / 2), sf + m * (K / 16));
    }
    free(v);
    return 0;
}

int orc_encode_colwise(const uint16_t* x, int64_t M, int64_t K, int64_t ld,
                       int per_vector, const float* amax, uint8_t* q, uint8_t* sf)
{
    if (M < 0 || K < 0 || M % 16 != 0) return -1;
    float* v = (float*)malloc(sizeof(float) * (size_t)(M > 0 ? M : 1));
    for (int64_t k = 0; k < K; ++k) {
        for (int64_t m = 0; m < M; ++m) v[m] = orc_bf16_to_f32(x[m * ld + k]);
        float A = per_vector ? amax[k] : amax[0];
        orc_quantize_vector(v, M, A, q + k * (M / 2), sf + k * (M / 16));
    }
    free(v);
    return 0;
}

/* 16x16 tiles: one E4M3 code per tile relative to the per-tensor outer
 * scale, so the rowwise and columnwise codes are the same numbers; emitted
 * in the per-token layout (scale replicated along each row / column of the
 * tile, amax vectors filled with the tensor amax).  Follows the opt-in 2D
 * weight mode described in the "Changes" list of the per-token recipe page. */
static int quantize_2d(const uint16_t* x, int64_t M, int64_t K,
                       uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                       uint8_t* col_q, uint8_t* col_sf, float* col_amax)
{
    if (M % 16 != 0 || K % 16 != 0) return -1;
    float A = orc_amax_tensor(x, M, K, K);
    float S = A / kOuterDiv;
    int64_t TI = M / 16, TJ = K / 16;
    for (int64_t I = 0; I < TI; ++I) {
        for (int64_t J = 0; J < TJ; ++J) {
            float tile[16][16];
            for (int a = 0; a < 16; ++a)
                for (int b = 0; b < 16; ++b)
                    tile[a][b] = orc_bf16_to_f32(x[(16 * I + a) * K + 16 * J + b]);
            uint8_t code;
            float r;
            if (S == 0.0f) {
                code = 0x00;
                r = 0.0f;
            } else {
                float bmax = 0.0f;
                for (int a = 0; a < 16; ++a)
                    for (int b = 0; b < 16; ++b) {
                        float m = fabsf(tile[a][b]);
                        if (m > bmax) bmax = m;
                    }
                float t = bmax / kE2M1Max;
                float s = t / S;
                code = orc_e4m3_encode(s);
                r = orc_e4m3_decode(code) * S;
            }
            uint8_t nib[16][16];
            for (int a = 0; a < 16; ++a) encode_block(tile[a], 16, r, nib[a]);
            for (int a = 0; a < 16; ++a) {
                int64_t m = 16 * I + a;
                for (int b = 0; b < 16; b += 2) {
                    int64_t k = 16 * J + b;
                    if (row_q) row_q[m * (K / 2) + k / 2] = (uint8_t)(nib[a][b] | (nib[a][b + 1] << 4));
                }
                if (row_sf) row_sf[m * (K / 16) + J] = code;
            }
            for (int b = 0; b < 16; ++b) {
                int64_t k = 16 * J + b;
                for (int a = 0; a < 16; a += 2) {
                    int64_t m = 16 * I + a;
                    if (col_q) col_q[k * (M / 2) + m / 2] = (uint8_t)(nib[a][b] | (nib[a + 1][b] << 4));
                }
                if (col_sf) col_sf[k * (M / 16) + I] = code;
            }
        }
    }
    if (row_amax) for (int64_t m = 0; m < M; ++m) row_amax[m] = A;
    if (col_amax) for (int64_t k = 0; k < K; ++k) col_amax[k] = A;
    return 0;
}

int orc_quantize(const uint16_t* x, int64_t M, int64_t K, int mode,
                 uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                 uint8_t* col_q, uint8_t* col_sf, float* col_amax)
{
    int want_row = row_q != NULL, want_col = col_q != NULL;
    if (M < 0 || K < 0) return -1;
    if (want_row && K % 16 != 0) return -1;
    if (want_col && M % 16 != 0) return -1;
    if (mode == 2)
        return quantize_2d(x, M, K, row_q, row_sf, row_amax, col_q, col_sf, col_amax);
    if (mode == 0) {
        /* per-tensor: one outer amax for the whole tensor (the recipe's default) */
        float A = orc_amax_tensor(x, M, K, K);
        if (want_row) {
            if (row_amax) row_amax[0] = A;
            orc_encode_rowwise(x, M, K, K, 0, &A, row_q, row_sf);
        }
        if (want_col) {
            if (col_amax) col_amax[0] = A;
            orc_encode_colwise(x, M, K, K, 0, &A, col_q, col_sf);
        }
        return 0;
    }
    if (mode == 1) {
        /* per-token: a per-row amax (length M) for rowwise data and a per-col
         * amax (length K) for columnwise data */
        if (want_row) {
            float* ra = (float*)malloc(sizeof(float) * (size_t)(M > 0 ? M : 1));
            orc_amax_rows(x, M, K, K, ra);
            orc_encode_rowwise(x, M, K, K, 1, ra, row_q, row_sf);
            if (row_amax) memcpy(row_amax, ra, sizeof(float) * (size_t)M);
            free(ra);
        }
        if (want_col) {
            float* ca = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
            orc_amax_cols(x, M, K, K, ca);
            orc_encode_colwise(x, M, K, K, 1, ca, col_q, col_sf);
            if (col_amax) memcpy(col_amax, ca, sizeof(float) * (size_t)K);
            free(ca);
        }
        return 0;
    }
    return -1;
}

int orc_quantize_grouped(const uint16_t* x, int64_t K, int32_t G, const int64_t* counts,
                         uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                         uint8_t* col_q, uint8_t* col_sf, float* col_amax)
{
    int64_t total = 0;
    for (int32_t e = 0; e < G; ++e) {
        if (counts[e] < 0 || counts[e] % 16 != 0) return -1;
        total += counts[e];
    }
    if (row_q) {
        if (K % 16 != 0) return -1;
        /* rowwise: per-token rowwise of the concatenated experts */
        if (orc_quantize(x, total, K, 1, row_q, row_sf, row_amax, NULL, NULL, NULL) != 0) return -1;
    }
    if (col_q) {
        int64_t off = 0;
        for (int32_t e = 0; e < G; ++e) {
            int64_t me = counts[e];
            const uint16_t* xe = x + off * K;
            float* ca = col_amax + (int64_t)e * K;
            orc_amax_cols(xe, me, K, K, ca);   /* an empty expert gives 0 */
            orc_encode_colwise(xe, me, K, K, 1, ca, col_q + K * off / 2, col_sf + K * off / 16);
            off += me;
        }
    }
    return 0;
}

/* ----------------------------------------------------------- dequantize */

int orc_dequantize(const uint8_t* q, const uint8_t* sf, const float* amax,
                   int64_t R, int64_t C, int amax_per_row, float* out)
{
    if (R < 0 || C < 0 || C % 16 != 0) return -1;
    for (int64_t r = 0; r < R; ++r) {
        float A = amax_per_row ? amax[r] : amax[0];
        float S = A / kOuterDiv;
        for (int64_t j = 0; j < C / 16; ++j) {
            float ratio = orc_e4m3_decode(sf[r * (C / 16) + j]) * S;
            for (int i = 0; i < 16; ++i) {
                int64_t c = 16 * j + i;
                uint8_t byte = q[r * (C / 2) + c / 2];
                uint8_t nib = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);
                float val = kE2M1[nib & 7] * ratio;
                out[r * C + c] = (nib & 8) ? -val : val;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------ decayed accumulate */

/* New = max(Old * Decay, Observed), from the PTQ scaling-factor buffering
 * page (TransformerEngine PR #3296, "Description"): decay 0 keeps only the
 * latest value, decay 1 keeps the maximum over the whole history. */
void orc_amax_accumulate(float* buf, const float* obs, int64_t n, float decay)
{
    for (int64_t i = 0; i < n; ++i) {
        float t = buf[i] * decay;
        buf[i] = (obs[i] > t) ? obs[i] : t;
    }
}

/* the same page max-reduces the row-wise vector to a scalar before it is
 * kept; an empty vector observes 0 */
void orc_amax_accumulate_reduce(float* buf, const float* obs, int64_t n, float decay)
{
    float m = 0.0f;
    for (int64_t i = 0; i < n; ++i)
        if (obs[i] > m) m = obs[i];
    orc_amax_accumulate(buf, &m, 1, decay);
}

/* --------------------------------------------------- stochastic rounding */

/* The per-token recipe page lists a stochastic-rounding variant of the cast
 * ("per_token_sr") without saying how its random numbers are drawn.  The
 * reading taken here (and in the design notes):
 *   - randoms come from Philox4x32-10, the counter-based generator of
 *     Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as
 *     1, 2, 3" (SC'11).  Key = the caller's 64-bit seed (low word first);
 *     element i of a vector (a row for rowwise output, a column for
 *     columnwise output) takes byte i % 16 of the block with counter
 *     (i / 16, vector index, direction, offset), the block's four output
 *     words read as 16 little-endian bytes (byte k = bits 8(k % 4) ..
 *     8(k % 4) + 7 of word k / 4); direction 0 rowwise and 1 columnwise,
 *     offset a 32-bit value the caller changes per call.  One block thus
 *     serves one 16-element block of the cast, eight random bits per element;
 *   - rounding: block scales exactly as in the deterministic cast; the
 *     element quotient x = |RN(v / r)| also; lo and lo + d the E2M1 grid
 *     points around x (d = 0.5 below 2, 1 below 4, 2 below 6); with
 *     U = R * 2^-8 for the element's 8-bit random R, the magnitude rounds up
 *     iff x - lo > U * d.  Both sides of that comparison are exact in
 *     binary32 (x - lo by Sterbenz's lemma, U * d a power-of-two scaling), so
 *     P(up) = ceil(2^8 * (x - lo) / d) / 2^8: the rounding's mean exceeds x
 *     by less than d / 256.  x >= 6 saturates to 6 with no draw; the sign is
 *     copied; r == 0 gives sign-only nibbles. */

/* One Philox4x32 block: ten rounds of the multiply-xor S-box on the counter
 * words, with the key advanced by the two Weyl constants between rounds. */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    const uint32_t kMul0 = 0xD2511F53u, kMul1 = 0xCD9E8D57u;   /* round multipliers */
    const uint32_t kWeyl0 = 0x9E3779B9u, kWeyl1 = 0xBB67AE85u; /* key increments */
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += kWeyl0;
            k1 += kWeyl1;
        }
        uint64_t p0 = (uint64_t)kMul0 * c0;
        uint64_t p1 = (uint64_t)kMul1 * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

void orc_philox4x32_10_array(const uint32_t* ctr, const uint32_t* key, int64_t n, uint32_t* out)
{
    for (int64_t i = 0; i < n; ++i) orc_philox4x32_10(ctr + 4 * i, key + 2 * i, out + 4 * i);
}

/* E2M1 code of q rounded stochastically with the 8-bit random rnd */
uint8_t orc_e2m1_encode_sr(float q, uint8_t rnd)
{
    uint8_t s = signbit(q) ? 8 : 0;
    float x = fabsf(q);
    if (x >= 6.0f) return (uint8_t)(s | 7);
    float lo, d;
    uint8_t c;
    if (x < 2.0f) {            /* grid 0, 0.5, 1, 1.5: codes 0..3 */
        c = (uint8_t)floorf(2.0f * x);
        lo = 0.5f * (float)c;
        d = 0.5f;
    } else if (x < 4.0f) {     /* grid 2, 3: codes 4, 5 */
        lo = floorf(x);
        c = (uint8_t)(2 + (int)lo);
        d = 1.0f;
    } else {                   /* grid 4: code 6, next 6 */
        lo = 4.0f;
        c = 6;
        d = 2.0f;
    }
    float u = (float)rnd * 0x1p-8f;
    if (x - lo > u * d) c = (uint8_t)(c + 1);
    return (uint8_t)(s | c);
}

void orc_e2m1_encode_sr_array(const float* q, const uint8_t* rnd, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_encode_sr(q[i], rnd[i]);
}

/* one vector, as orc_quantize_vector, with stochastic element rounding */
void orc_quantize_vector_sr(const float* v, int64_t n, float A, uint8_t* q, uint8_t* sf,
                            uint64_t seed, uint32_t vec, uint32_t dir, uint32_t offset)
{
    float S = A / kOuterDiv;
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    for (int64_t j = 0; j < n / 16; ++j) {
        const float* blk = v + 16 * j;
        float r;
        if (S == 0.0f) {
            sf[j] = 0x00;
            r = 0.0f;
        } else {
            float b = 0.0f;
            for (int i = 0; i < 16; ++i) {
                float a = fabsf(blk[i]);
                if (a > b) b = a;
            }
            float t = b / kE2M1Max;
            float s = t / S;
            uint8_t code = orc_e4m3_encode(s);
            sf[j] = code;
            r = orc_e4m3_decode(code) * S;
        }
        /* elements 16 j .. 16 j + 15: bytes 0 .. 15 of block (j, vec, dir, offset) */
        uint32_t words[4];
        uint32_t ctr[4] = {(uint32_t)j, vec, dir, offset};
        orc_philox4x32_10(ctr, key, words);
        uint8_t nib[16];
        for (int i = 0; i < 16; ++i) {
            uint8_t rnd = (uint8_t)(words[i / 4] >> (8 * (i % 4)));
            if (r == 0.0f)
                nib[i] = signbit(blk[i]) ? 8 : 0;
            else
                nib[i] = orc_e2m1_encode_sr(blk[i] / r, rnd);
        }
        for (int i = 0; i < 8; ++i)
            q[8 * j + i] = (uint8_t)(nib[2 * i] | (nib[2 * i + 1] << 4));
    }
}

/* whole stochastic-rounding cast, per-tensor (mode 0) or per-token (mode 1);
 * amax outputs as orc_quantize.  M < 2^32 (the vector index is one counter
 * word).  Returns 0, or -1 on a shape or mode error. */
int orc_quantize_sr(const uint16_t* x, int64_t M, int64_t K, int mode,
                    uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                    uint8_t* col_q, uint8_t* col_sf, float* col_amax,
                    uint64_t seed, uint32_t offset)
{
    int want_row = row_q != NULL, want_col = col_q != NULL;
    if (M < 0 || K < 0 || M >= ((int64_t)1 << 32) || (mode != 0 && mode != 1)) return -1;
    if (want_row && K % 16 != 0) return -1;
    if (want_col && M % 16 != 0) return -1;
    float At = mode == 0 ? orc_amax_tensor(x, M, K, K) : 0.0f;
    if (want_row) {
        float* ra = (float*)malloc(sizeof(float) * (size_t)(M > 0 ? M : 1));
        float* v = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
        if (mode == 1) orc_amax_rows(x, M, K, K, ra);
        for (int64_t m = 0; m < M; ++m) {
            for (int64_t k = 0; k < K; ++k) v[k] = orc_bf16_to_f32(x[m * K + k]);
            orc_quantize_vector_sr(v, K, mode == 1 ? ra[m] : At, row_q + m * (K / 2), row_sf + m * (K / 16),
                                   seed, (uint32_t)m, 0u, offset);
        }
        if (row_amax) {
            if (mode == 1) memcpy(row_amax, ra, sizeof(float) * (size_t)M);
            else row_amax[0] = At;
        }
        free(v);
        free(ra);
    }
    if (want_col) {
        float* ca = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
        float* v = (float*)malloc(sizeof(float) * (size_t)(M > 0 ? M : 1));
        if (mode == 1) orc_amax_cols(x, M, K, K, ca);
        for (int64_t k = 0; k < K; ++k) {
            for (int64_t m = 0; m < M; ++m) v[m] = orc_bf16_to_f32(x[m * K + k]);
            orc_quantize_vector_sr(v, M, mode == 1 ? ca[k] : At, col_q + k * (M / 2), col_sf + k * (M / 16),
                                   seed, (uint32_t)k, 1u, offset);
        }
        if (col_amax) {
            if (mode == 1) memcpy(col_amax, ca, sizeof(float) * (size_t)K);
            else col_amax[0] = At;
        }
        free(v);
        free(ca);
    }
    return 0;
}

/* ------------------------------------------------------ GEMM consumer */

/* The per-token recipe page's GEMM consumer ("Changes": a GEMM that rescales
 * with the per-row / per-col outer-amax vectors inside its epilogue; the
 * sequence diagram's nvfp4_cutlass_per_token_gemm(A_data, A_sf, A_row_amax,
 * B_data, B_sf, B_col_amax) -> output (M, N)), written for two NVFP4
 * operands whose 16-element blocks run along the contraction dimension K:
 *   out[m][n] = S_a(m) * S_b(n) * sum_k (g_a * D_a)[m][k] * (g_b * D_b)[n][k]
 * with g the E2M1 value, D the decoded E4M3 block scale and S = RN(amax /
 * 2688), per row (per_row = 1) or one per tensor.  The forward (TN), dgrad
 * (NN) and wgrad (NT) products of the page are this form applied to the
 * rowwise or columnwise output of the cast.  Computed here in binary64:
 * each product of block values is exact, the sum over K rounds at most
 * once per term at 2^-53, then the two outer scales.  bound[m][n] (may be
 * NULL) receives S_a * S_b * sum_k |term|, the magnitude error bounds of a
 * binary32 evaluation scale with. */
static double deq_block_value(const uint8_t* q, const uint8_t* sf, int64_t row, int64_t K, int64_t k)
{
    uint8_t byte = q[row * (K / 2) + k / 2];
    uint8_t nib = (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
    return (double)orc_e2m1_decode(nib) * (double)orc_e4m3_decode(sf[row * (K / 16) + k / 16]);
}

int orc_gemm_nvfp4(const uint8_t* aq, const uint8_t* asf, const float* aamax, int a_per_row,
                   const uint8_t* bq, const uint8_t* bsf, const float* bamax, int b_per_row,
                   int64_t M, int64_t N, int64_t K, double* out, double* bound)
{
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0) return -1;
    double* a = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k) a[k] = deq_block_value(aq, asf, m, K, k);
        double sa = (double)(aamax[a_per_row ? m : 0] / kOuterDiv);
        for (int64_t n = 0; n < N; ++n) {
            double sb = (double)(bamax[b_per_row ? n : 0] / kOuterDiv);
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double t = a[k] * deq_block_value(bq, bsf, n, K, k);
                acc += t;
                mag += fabs(t);
            }
            out[m * N + n] = acc * sa * sb;
            if (bound) bound[m * N + n] = mag * sa * sb;
        }
    }
    free(a);
    return 0;
}

/* ------------------------------------------ random Hadamard transform */

/* The per-token recipe page lists a random Hadamard transform as an opt-in
 * for the columnwise direction only (PR #3045, "Changes": per_token_rht, and
 * the review's note that the row direction never uses it).  The pages fix
 * neither its size nor its arithmetic; the readings taken here:
 *   - size 16, one transform per 16-element block of a columnwise vector
 *     (the block the E4M3 scale covers);
 *   - y = (1/4) H16 D x with H16 the Sylvester Hadamard matrix,
 *     H16[i][j] = (-1)^popcount(i & j), and D = diag(s), s_j = -1 where bit j
 *     of a caller-given 16-bit sign mask is set, else +1;
 *   - evaluated in binary32 as the fast Walsh-Hadamard butterfly: stages
 *     h = 1, 2, 4, 8, each replacing the pair (v[i], v[i+h]), i & h == 0, by
 *     (v[i] + v[i+h], v[i] - v[i+h]); then times 1/4 (exact for normal
 *     results) and rounded to bf16, nearest-even.
 * The transformed bf16 block then goes through the ordinary cast.  Natural
 * (Sylvester) ordering: the butterfly above yields y_i = sum_j H16[i][j]
 * s_j x_j / 4 up to binary32 rounding. */
static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

void orc_rht16(const uint16_t in[16], uint32_t sign_mask, uint16_t out[16])
{
    float v[16];
    for (int j = 0; j < 16; ++j) {
        v[j] = orc_bf16_to_f32(in[j]);
        if ((sign_mask >> j) & 1u) v[j] = -v[j];
    }
    for (int h = 1; h < 16; h <<= 1)
        for (int i = 0; i < 16; ++i)
            if (!(i & h)) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
    for (int j = 0; j < 16; ++j) out[j] = f32_to_bf16_rne(v[j] * 0.25f);
}

/* y [M][K] = the transform applied down each column of x [M][K] (M % 16 == 0),
 * block by block of 16 rows */
int orc_rht_columns(const uint16_t* x, int64_t M, int64_t K, uint32_t sign_mask, uint16_t* y)
{
    if (M < 0 || K < 0 || M % 16 != 0) return -1;
    uint16_t in[16], out[16];
    for (int64_t r0 = 0; r0 < M; r0 += 16)
        for (int64_t k = 0; k < K; ++k) {
            for (int i = 0; i < 16; ++i) in[i] = x[(r0 + i) * K + k];
            orc_rht16(in, sign_mask, out);
            for (int i = 0; i < 16; ++i) y[(r0 + i) * K + k] = out[i];
        }
    return 0;
}

/* -------------------------------------------- GEMM-swizzled scale layout */

/* The per-token recipe page keeps block scales unswizzled
 * (with_gemm_swizzled_scales off, with_swizzle=0) and leaves the swizzled
 * layout to the GEMM consumer; the pages do not define it.  Reading: the
 * tiled layout block-scaled GEMMs take for 16-element FP4 blocks, written
 * here from its definition.  For a scale matrix sf [R][nb] (row r, block c):
 *   Rp = R rounded up to 128, nbp = nb rounded up to 4;
 *   tiles of 128 rows x 4 blocks, 512 bytes each, row-tile major:
 *     tile(r, c) = (r / 128) * (nbp / 4) + c / 4
 *   inside a tile, row r lands in 16-byte line r % 32 at 4-byte slot
 *   (r / 32) % 4, block c at byte c % 4 of the slot:
 *     offset(r, c) = 512 * tile(r, c) + 16 * (r % 32) + 4 * ((r / 32) % 4) + c % 4
 * Bytes of the Rp * nbp layout that no (r < R, c < nb) maps to are zero. */
int64_t orc_swizzled_size(int64_t R, int64_t nb)
{
    return ((R + 127) / 128 * 128) * ((nb + 3) / 4 * 4);
}

int orc_swizzle_scales(const uint8_t* sf, int64_t R, int64_t nb, uint8_t* out)
{
    if (R < 0 || nb < 0) return -1;
    const int64_t nbp = (nb + 3) / 4 * 4;
    memset(out, 0, (size_t)orc_swizzled_size(R, nb));
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < nb; ++c) {
            int64_t tile = (r / 128) * (nbp / 4) + c / 4;
            int64_t off = 512 * tile + 16 * (r % 32) + 4 * ((r / 32) % 4) + c % 4;
            out[off] = sf[r * nb + c];
        }
    return 0;
}

int orc_unswizzle_scales(const uint8_t* in, int64_t R, int64_t nb, uint8_t* sf)
{
    if (R < 0 || nb < 0) return -1;
    const int64_t nbp = (nb + 3) / 4 * 4;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < nb; ++c) {
            int64_t tile = (r / 128) * (nbp / 4) + c / 4;
            sf[r * nb + c] = in[512 * tile + 16 * (r % 32) + 4 * ((r / 32) % 4) + c % 4];
        }
    return 0;
}


/* ---- CPU baseline driver: the per-token row + column cast above, with the
 * rows and the columns partitioned over threads.  Each thread runs the same
 * per-vector routines (orc_amax_rows / orc_encode_rowwise on its rows,
 * orc_amax_cols / orc_encode_colwise on its columns); nothing is blocked,
 * fused or reordered beyond that split.  Used to time the oracle on the
 * host's cores. */
struct orc_slice {
    const uint16_t* x;
    int64_t M, K, r0, r1, c0, c1;
    uint8_t *row_q, *row_sf, *col_q, *col_sf;
    float *row_amax, *col_amax;
};

static void* orc_slice_run(void* arg)
{
    struct orc_slice* a = (struct orc_slice*)arg;
    const int64_t M = a->M, K = a->K;
    if (a->row_q && a->r1 > a->r0) {
        orc_amax_rows(a->x + a->r0 * K, a->r1 - a->r0, K, K, a->row_amax + a->r0);
        orc_encode_rowwise(a->x + a->r0 * K, a->r1 - a->r0, K, K, 1, a->row_amax + a->r0,
                           a->row_q + a->r0 * (K / 2), a->row_sf + a->r0 * (K / 16));
    }
    if (a->col_q && a->c1 > a->c0) {
        orc_amax_cols(a->x + a->c0, M, a->c1 - a->c0, K, a->col_amax + a->c0);
        orc_encode_colwise(a->x + a->c0, M, a->c1 - a->c0, K, 1, a->col_amax + a->c0,
                           a->col_q + a->c0 * (M / 2), a->col_sf + a->c0 * (M / 16));
    }
    return NULL;
}

int orc_quantize_per_token_threads(const uint16_t* x, int64_t M, int64_t K, int nthreads,
                                   uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                                   uint8_t* col_q, uint8_t* col_sf, float* col_amax)
{
    if (M < 0 || K < 0 || nthreads < 1 || nthreads > 1024) return -1;
    if (row_q && K % 16 != 0) return -1;
    if (col_q && M % 16 != 0) return -1;
    struct orc_slice* sl = (struct orc_slice*)calloc((size_t)nthreads, sizeof(struct orc_slice));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!sl || !th) { free(sl); free(th); return -1; }
    for (int i = 0; i < nthreads; ++i) {
        struct orc_slice* a = &sl[i];
        a->x = x; a->M = M; a->K = K;
        a->r0 = M * i / nthreads; a->r1 = M * (i + 1) / nthreads;
        a->c0 = K * i / nthreads; a->c1 = K * (i + 1) / nthreads;
        a->row_q = row_q; a->row_sf = row_sf; a->row_amax = row_amax;
        a->col_q = col_q; a->col_sf = col_sf; a->col_amax = col_amax;
    }
    int started = 0, rc = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, orc_slice_run, &sl[i]) != 0) { rc = -1; break; }
        started = i;
    }
    orc_slice_run(&sl[0]);
    for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
    if (rc == 0) {
        /* any slice a failed thread would have covered, done here */
        for (int i = started + 1; i < nthreads; ++i) orc_slice_run(&sl[i]);
    }
    free(sl);
    free(th);
    return 0;
}
