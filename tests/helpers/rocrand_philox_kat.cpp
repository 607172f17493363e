// Known-answer generator for Philox4x32-10 from an independent implementation: rocRAND's
// host-callable philox4x32_10_engine.  Reads lines "c0 c1 c2 c3 k0 k1" (hex) on stdin and
// prints the four output words of the block with that counter and key.  The engine takes the
// key as the seed, counter words 2-3 as the subsequence and counter words 0-1 (times 4) as the
// offset, so counter word 1 must stay below 2^30 here.
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

int main() {
    unsigned c0, c1, c2, c3, k0, k1;
    while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        unsigned long long seed = ((unsigned long long)k1 << 32) | k0;
        unsigned long long subseq = ((unsigned long long)c3 << 32) | c2;
        unsigned long long offset = 4ull * (((unsigned long long)c1 << 32) | c0);
        rocrand_device::philox4x32_10_engine eng(seed, subseq, offset);
        unsigned a = eng(), b = eng(), c = eng(), d = eng();
        std::printf("%08x %08x %08x %08x\n", a, b, c, d);
    }
    return 0;
}
