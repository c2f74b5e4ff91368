/* The fast path's E4M3 code for a block scale sf in the subnormal range
 * (0 < sf < 2^-6; nvfp4_device.hpp, fast_block with SUB): m = the bits of
 * sf * 2^9 + 2^23 less those of 2^23, i.e. RNE(sf * 2^9) (sf * 2^9 < 8 is
 * exact, and at 2^23 the float spacing is 1, so the addition rounds to the
 * nearest integer, ties to even), and its value m * 2^-9.  Compared with the
 * oracle's E4M3 encoder and decoder (oracle/nvfp4_oracle.c) for every fp32
 * bit pattern in that range.  Prints "<n> checked, <m> mismatches". */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

uint8_t orc_e4m3_encode(float s);
float orc_e4m3_decode(uint8_t code);

static float f_of(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t b_of(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

int main(void)
{
    uint64_t n = 0, m_bad = 0;
    for (uint32_t u = 1; u < 0x3C800000u; ++u) {
        const float sf = f_of(u);
        const uint32_t m = b_of(sf * 512.0f + 8388608.0f) - 0x4B000000u;
        const uint8_t c = orc_e4m3_encode(sf);
        ++n;
        if (m != c || (float)m * 0x1p-9f != orc_e4m3_decode(c)) {
            if (m_bad < 3) printf("mismatch sf=%08x kernel %u oracle %u\n", u, m, c);
            ++m_bad;
        }
    }
    printf("%llu checked, %llu mismatches\n", (unsigned long long)n, (unsigned long long)m_bad);
    return m_bad != 0;
}
