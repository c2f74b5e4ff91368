/*
 * Exhaustive check of the division shortcut used by the HIP encode kernels.
 *
 * The kernels need q = RN(a / r) for every element a (a bf16 value widened
 * to fp32) of a block whose ratio r = D * S is shared by the block.  Instead
 * of one IEEE division per element they compute, per block, y = RN(1/r)
 * (one correctly rounded division) and per element
 *     q0 = RN(a * y)
 *     e  = RN(r * q0 - a)          (one fma; exact when q0 is close to a/r)
 *     q  = RN(q0 - e * y)          (one fma)
 * which is Markstein's correction step (P. Markstein, "Computation of
 * elementary functions on the IBM RISC System/6000 processor", IBM J. Res.
 * Dev. 34(1), 1990; also Muller et al., Handbook of Floating-Point
 * Arithmetic, the chapter on division with fused multiply-add).  The residual
 * is written as r*q0 - a (not a - r*q0) so that a = -0 keeps its sign.
 *
 * Claim checked here: q == RN(a / r) bit for bit for every bf16 significand
 * of a (both signs) and every fp32 significand of r.  A second family checks
 * the same sequence for the block-scale quotient sf = RN(t / S), whose
 * numerator t = RN(b / 6) (b bf16) takes only 128 distinct significands:
 * every one of them against every fp32 significand of S.  The three steps are
 * exact under scaling by powers of two while every intermediate is a normal
 * number, so one exponent pair covers the whole range the kernels allow
 * (r in [2^-64, 2^64] and |a| * y <= 2^64); the run also samples other
 * exponent pairs, tiny and subnormal a (where only the E2M1 code and its sign
 * must agree), and signed zeros.
 *
 * A third family checks the two-op element quotient the encode kernels use:
 * per block y_hi = RD(1/r) (RN(1/r), stepped down one ulp when r*y > 1) and
 * y_lo = RN((1 - r*y_hi) * y_hi) >= 0, per element q = fma(a, y_hi, a*y_lo).
 * It is not always RN(a/r) (it can differ in the last bit), so what is
 * checked is the E2M1 code of q against the code of RN(a/r), for every bf16
 * significand of a (both signs) against every significand of r, at the eight
 * exponent offsets that put a/r anywhere in [2^-4, 2^4] (below, both codes
 * are a signed zero; above, both saturate), plus tiny and zero numerators.
 * The one divisor significand where the codes can differ, all mantissa bits
 * set (r = 2^k * (2 - 2^-23), with a/r just above 0.25), is excluded here:
 * the kernels send blocks with such an r to the exact path.
 *
 * Build: gcc -O2 -mfma -ffp-contract=off -pthread; prints one summary line
 * and exits 0 only if nothing disagrees.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float shortcut(float a, float r, float y)
{
    float q0 = a * y;
    /* volatile keeps the compiler from moving the negation across the two
     * fmas, a rewrite that is not exact for signed zeros */
    volatile float e = fmaf(r, q0, -a);
    float ne = -e;
    return fmaf(ne, y, q0);
}

/* E2M1 code of a float (RNE onto 0,.5,1,1.5,2,3,4,6, saturating, sign copied) */
static unsigned e2m1(float q)
{
    unsigned s = signbit(q) ? 8u : 0u;
    float a = fabsf(q);
    unsigned c = a <= 0.25f ? 0 : a < 0.75f ? 1 : a <= 1.25f ? 2 : a < 1.75f ? 3
               : a <= 2.5f ? 4 : a < 3.5f ? 5 : a <= 5.0f ? 6 : 7;
    return s | c;
}

typedef struct { int task; uint64_t checked, bad; } job_t;

/* task in [0, 256): sign = task >> 7, bf16 significand m = task & 127 */
static void* run_exhaustive(void* p)
{
    job_t* j = (job_t*)p;
    uint32_t sign = (uint32_t)(j->task >> 7) << 31;
    uint32_t m = (uint32_t)(j->task & 127);
    /* exponent pairs: (0,0) exhaustively; a few others on every 13th r */
    static const int ea_list[] = {0, 5, -9, 20, -40};
    static const int er_list[] = {0, -3, 7, 44, -60};
    for (int p2 = 0; p2 < 5; ++p2) {
        uint32_t step = p2 == 0 ? 1 : 13;
        float a = f_of(sign | ((uint32_t)(127 + ea_list[p2]) << 23) | (m << 16));
        for (uint32_t mr = 0; mr < (1u << 23); mr += step) {
            float r = f_of(((uint32_t)(127 + er_list[p2]) << 23) | mr);
            float y = 1.0f / r;
            float q = shortcut(a, r, y);
            float ref = a / r;
            j->checked++;
            if (u_of(q) != u_of(ref)) {
                if (j->bad < 4)
                    fprintf(stderr, "mismatch a=%08x r=%08x got=%08x want=%08x\n",
                            u_of(a), u_of(r), u_of(q), u_of(ref));
                j->bad++;
            }
        }
    }
    return NULL;
}

/* two-op element quotient */
static float quot2(float a, float r)
{
    float y = 1.0f / r;
    volatile float e = fmaf(-r, y, 1.0f);
    float yhi = e < 0.0f ? f_of(u_of(y) - 1u) : y;
    volatile float e2 = fmaf(-r, yhi, 1.0f);
    float ylo = e2 * yhi;
    volatile float p = a * ylo;
    return fmaf(a, yhi, p);
}

static void* run_two_op(void* p)
{
    job_t* j = (job_t*)p;
    uint32_t sign = (uint32_t)(j->task >> 7) << 31;
    uint32_t m = (uint32_t)(j->task & 127);
    for (int ea = -3; ea <= 4; ++ea) {
        float a = f_of(sign | ((uint32_t)(127 + ea) << 23) | (m << 16));
        for (uint32_t mr = 0; mr < (1u << 23) - 1u; ++mr) {
            float r = f_of((127u << 23) | mr);
            float q = quot2(a, r), ref = a / r;
            j->checked++;
            if (e2m1(q) != e2m1(ref)) {
                if (j->bad < 4)
                    fprintf(stderr, "two-op mismatch a=%08x r=%08x got=%08x want=%08x\n",
                            u_of(a), u_of(r), u_of(q), u_of(ref));
                j->bad++;
            }
        }
    }
    return NULL;
}

/* block-scale family: t = RN(b/6) for the 128 bf16 significands of b in
 * [1, 2), divided by every significand of S in [1, 2) */
static void* run_scale_family(void* p)
{
    job_t* j = (job_t*)p;
    float b = f_of(((uint32_t)127 << 23) | ((uint32_t)j->task << 16));
    float t = b / 6.0f;
    for (uint32_t ms = 0; ms < (1u << 23); ++ms) {
        float S = f_of(((uint32_t)127 << 23) | ms);
        float y = 1.0f / S;
        float q = shortcut(t, S, y);
        float ref = t / S;
        j->checked++;
        if (u_of(q) != u_of(ref)) {
            if (j->bad < 4)
                fprintf(stderr, "scale mismatch t=%08x S=%08x got=%08x want=%08x\n",
                        u_of(t), u_of(S), u_of(q), u_of(ref));
            j->bad++;
        }
    }
    return NULL;
}

/* tiny and subnormal a against r at the ends of the allowed range: the
 * E2M1 code (magnitude and sign) must agree */
static void check_tiny(uint64_t* checked, uint64_t* bad)
{
    uint32_t seed = 12345u;
    for (uint32_t abits = 0; abits < 0x2000u; ++abits) {     /* bf16 with exponent field < 64 */
        for (int s = 0; s < 2; ++s) {
            float a = f_of(((uint32_t)s << 31) | (abits << 16));
            for (int k = 0; k < 64; ++k) {
                seed = seed * 1664525u + 1013904223u;
                int er = -64 + (int)(seed >> 25);          /* -64 .. 63 */
                seed = seed * 1664525u + 1013904223u;
                float r = f_of(((uint32_t)(127 + er) << 23) | (seed >> 9));
                float y = 1.0f / r;
                if (fabsf(a) * y > 0x1p64f) continue;
                float q = shortcut(a, r, y);
                float ref = a / r;
                (*checked)++;
                if (e2m1(q) != e2m1(ref)) {
                    if (*bad < 4)
                        fprintf(stderr, "tiny mismatch a=%08x r=%08x got=%08x want=%08x\n",
                                u_of(a), u_of(r), u_of(q), u_of(ref));
                    (*bad)++;
                }
            }
        }
    }
    /* the two-op quotient on tiny and subnormal numerators */
    for (uint32_t abits = 0; abits < 0x2000u; ++abits) {
        for (int s = 0; s < 2; ++s) {
            float a = f_of(((uint32_t)s << 31) | (abits << 16));
            for (int k = 0; k < 16; ++k) {
                seed = seed * 1664525u + 1013904223u;
                int er = -64 + (int)(seed >> 25);
                seed = seed * 1664525u + 1013904223u;
                float r = f_of(((uint32_t)(127 + er) << 23) | (seed >> 9));
                if (fabsf(a) / r > 0x1p64f || (u_of(r) & 0x7FFFFFu) == 0x7FFFFFu) continue;
                (*checked)++;
                if (e2m1(quot2(a, r)) != e2m1(a / r)) {
                    if (*bad < 4) fprintf(stderr, "two-op tiny mismatch a=%08x r=%08x\n", u_of(a), u_of(r));
                    (*bad)++;
                }
            }
        }
    }
    /* signed zeros */
    float rs[] = {0x1p-64f, 1.0f, 3.0f, 0x1.fffffep63f};
    for (int i = 0; i < 4; ++i) {
        float y = 1.0f / rs[i];
        float qp = shortcut(0.0f, rs[i], y), qn = shortcut(-0.0f, rs[i], y);
        (*checked) += 2;
        if (u_of(qp) != 0u || u_of(qn) != 0x80000000u) {
            fprintf(stderr, "signed zero lost for r=%a\n", (double)rs[i]);
            (*bad)++;
        }
        float zp = quot2(0.0f, rs[i]), zn = quot2(-0.0f, rs[i]);
        (*checked) += 2;
        if (u_of(zp) != 0u || u_of(zn) != 0x80000000u) {
            fprintf(stderr, "two-op signed zero lost for r=%a\n", (double)rs[i]);
            (*bad)++;
        }
    }
}

int main(void)
{
    enum { NT = 256 };
    static job_t jobs[NT];
    static pthread_t th[NT];
    uint64_t checked = 0, bad = 0;
    /* 256 tasks, at most 16 threads at a time */
    for (int base = 0; base < NT; base += 16) {
        for (int t = base; t < base + 16; ++t) {
            jobs[t].task = t; jobs[t].checked = 0; jobs[t].bad = 0;
            pthread_create(&th[t], NULL, run_exhaustive, &jobs[t]);
        }
        for (int t = base; t < base + 16; ++t) {
            pthread_join(th[t], NULL);
            checked += jobs[t].checked;
            bad += jobs[t].bad;
        }
    }
    for (int base = 0; base < 128; base += 16) {
        for (int t = base; t < base + 16; ++t) {
            jobs[t].task = t; jobs[t].checked = 0; jobs[t].bad = 0;
            pthread_create(&th[t], NULL, run_scale_family, &jobs[t]);
        }
        for (int t = base; t < base + 16; ++t) {
            pthread_join(th[t], NULL);
            checked += jobs[t].checked;
            bad += jobs[t].bad;
        }
    }
    for (int base = 0; base < NT; base += 16) {
        for (int t = base; t < base + 16; ++t) {
            jobs[t].task = t; jobs[t].checked = 0; jobs[t].bad = 0;
            pthread_create(&th[t], NULL, run_two_op, &jobs[t]);
        }
        for (int t = base; t < base + 16; ++t) {
            pthread_join(th[t], NULL);
            checked += jobs[t].checked;
            bad += jobs[t].bad;
        }
    }
    check_tiny(&checked, &bad);
    printf("checked %llu cases, %llu mismatches\n", (unsigned long long)checked, (unsigned long long)bad);
    return bad == 0 ? 0 : 1;
}
