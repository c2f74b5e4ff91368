// Host program for the oracle's Philox4x32-10 pin: reads lines of six
// decimal words "c0 c1 c2 c3 k0 k1" and prints the four output words of
// rocRAND's Philox4x32-10 block function for that counter and key (the
// engine's ten-round function, protected there and re-exported by a derived
// class; only host code runs here).
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

struct Block : rocrand_device::philox4x32_10_engine {
    using rocrand_device::philox4x32_10_engine::ten_rounds;
};

int main() {
    Block engine;
    unsigned c0, c1, c2, c3, k0, k1;
    while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        const uint4 r = engine.ten_rounds(uint4{c0, c1, c2, c3}, uint2{k0, k1});
        std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
