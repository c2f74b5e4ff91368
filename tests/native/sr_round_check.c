/* The stochastic E2M1 rounding of the SR encoding kernel (nvfp4_kernels.hip,
 * e2m1_sr: a branch-free form on the bits of |q|) against the oracle's rule
 * (orc_e2m1_encode_sr), for every fp32 bit pattern q that is not a NaN, each
 * with an 8-bit random drawn from a hash of q.  The two forms compute the
 * same two exact binary32 values x - lo and U*d wherever they pick the same
 * (lo, d, code), so one random per q checks the pick; the hash still varies
 * which side of the threshold each q falls.  Then every random value for a
 * dense set of q (see main) and at the grid points, midpoints and their
 * neighbours.  Prints "<n> checked, <m>
 * mismatches". */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

uint8_t orc_e2m1_encode_sr(float q, uint8_t rnd);

static float f_of(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }

/* the kernel's form, transcribed (rnd: the element's 8-bit random) */
static uint32_t kernel_sr(float q, uint32_t rnd)
{
    uint32_t b;
    memcpy(&b, &q, 4);
    const uint32_t xb = b & 0x7fffffffu;
    const uint32_t ta = xb - 0x3f000000u;
    const uint32_t tb = (uint32_t)ceilf(f_of(xb < 0x3f800000u ? xb : 0x3f800000u) * 0x1p23f);
    const uint32_t t = xb >= 0x3f800000u ? ta : tb;
    const uint32_t r24 = (rnd & 0xffu) << 24;
    const uint32_t c = (t >> 22) + ((t << 10) > r24 ? 1u : 0u);
    return ((b >> 28) & 8u) | (c < 7u ? c : 7u);
}

static uint32_t hash(uint32_t x)
{
    x ^= x >> 16; x *= 0x7feb352dU; x ^= x >> 15; x *= 0x846ca68bU; x ^= x >> 16;
    return x;
}

#define NT 8
static uint64_t bad[NT], seen[NT];

static void* work(void* arg)
{
    const int t = (int)(intptr_t)arg;
    for (uint64_t i = (uint64_t)t; i < ((uint64_t)1 << 32); i += NT) {
        const uint32_t b = (uint32_t)i;
        if ((b & 0x7fffffffu) > 0x7f800000u) continue;   /* NaN */
        const float q = f_of(b);
        const uint8_t rnd = (uint8_t)(hash(b) >> 24);
        ++seen[t];
        if (kernel_sr(q, rnd) != orc_e2m1_encode_sr(q, rnd)) {
            if (bad[t] < 3) printf("mismatch q=%08x rnd=%08x kernel %u oracle %u\n", b, rnd, kernel_sr(q, rnd),
                                   orc_e2m1_encode_sr(q, rnd));
            ++bad[t];
        }
    }
    return NULL;
}

int main(void)
{
    pthread_t th[NT];
    for (int t = 0; t < NT; ++t) pthread_create(&th[t], NULL, work, (void*)(intptr_t)t);
    uint64_t n = 0, m = 0, m_all = 0;
    for (int t = 0; t < NT; ++t) {
        pthread_join(th[t], NULL);
        n += seen[t];
        m += bad[t];
    }
    /* every random value for: every q whose mantissa has at most its top 9
       bits set (its position between grid neighbours is then a multiple of
       1/256 of a step at most binades, where ties with U*d fall), and every
       97th mantissa of the binades from 2^-30 up to 8, both signs */
    for (uint32_t e = 0; e < 256; ++e)
        for (uint32_t m = 0; m < 512; ++m)
            for (uint32_t sg = 0; sg < 2; ++sg) {
                const uint32_t bb = (sg << 31) | (e << 23) | (m << 14);
                if ((bb & 0x7fffffffu) > 0x7f800000u) continue;
                for (uint32_t r = 0; r < 256; ++r) {
                    ++n;
                    if (kernel_sr(f_of(bb), r) != orc_e2m1_encode_sr(f_of(bb), (uint8_t)r)) ++m_all;
                }
            }
    for (uint32_t e = 97; e < 130; ++e)
        for (uint32_t m = 0; m < (1u << 23); m += 97)
            for (uint32_t sg = 0; sg < 2; ++sg) {
                const uint32_t bb = (sg << 31) | (e << 23) | m;
                for (uint32_t r = 0; r < 256; ++r) {
                    ++n;
                    if (kernel_sr(f_of(bb), r) != orc_e2m1_encode_sr(f_of(bb), (uint8_t)r)) ++m_all;
                }
            }
    m += m_all;
    /* every random value at the grid's points, midpoints, ends and their
       neighbours */
    const float pts[] = {0.0f, 0.25f, 0.5f, 0.75f, 1.0f, 1.25f, 1.5f, 1.75f, 2.0f, 2.5f, 3.0f, 3.5f, 4.0f, 5.0f, 6.0f,
                         5.9999995f, 1.9999999f, 0.49999997f, 0.99999994f, 0.25000003f, 2.5000002f, 4.9999995f};
    for (size_t i = 0; i < sizeof pts / sizeof pts[0]; ++i)
        for (uint32_t r = 0; r < 256; ++r)
            for (int sg = 0; sg < 2; ++sg) {
                const float q = sg ? -pts[i] : pts[i];
                ++n;
                if (kernel_sr(q, r) != orc_e2m1_encode_sr(q, (uint8_t)r)) ++m;
            }
    printf("%llu checked, %llu mismatches\n", (unsigned long long)n, (unsigned long long)m);
    return m != 0;
}
