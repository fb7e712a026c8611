// Known-answer source for Philox4x32-10: runs rocRAND's Philox engine on the
// host (the library is used as a black box) for arbitrary key and counter
// words.  Reads lines "k0 k1 c0 c1 c2 c3" (hex) from stdin and prints the
// four output words (hex) of one Philox4x32-10 block per line.
//
// rocRAND's engine keys with (seed lo, seed hi) and starts its counter at
// (0, 0, subsequence lo, subsequence hi); skipping ahead by 4*n values adds
// n to the low 64 bits of the counter.  So counter (c0, c1, c2, c3) is
// reached with seed = k0 | k1 << 32, subsequence = c2 | c3 << 32 and a skip
// of 4 * (c0 | c1 << 32), done in pieces that do not overflow.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

int main()
{
    unsigned k0, k1, c0, c1, c2, c3;
    while (std::scanf("%x %x %x %x %x %x", &k0, &k1, &c0, &c1, &c2, &c3) == 6) {
        rocrand_state_philox4x32_10 st;
        unsigned long long seed = (unsigned long long)k0 | ((unsigned long long)k1 << 32);
        unsigned long long sub = (unsigned long long)c2 | ((unsigned long long)c3 << 32);
        rocrand_init(seed, sub, 0ull, &st);
        unsigned long long lowctr = (unsigned long long)c0 | ((unsigned long long)c1 << 32);
        const unsigned long long piece = 1ull << 60;
        while (lowctr > 0) {
            unsigned long long step = lowctr > piece ? piece : lowctr;
            skipahead(4ull * step, &st);
            lowctr -= step;
        }
        unsigned a = rocrand(&st), b = rocrand(&st), c = rocrand(&st), d = rocrand(&st);
        std::printf("%08x %08x %08x %08x\n", a, b, c, d);
    }
    return 0;
}
