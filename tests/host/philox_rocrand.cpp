// philox_rocrand.cpp -- an independent Philox4x32-10 (Salmon et al., SC'11)
// for pinning the oracle's generator: rocRAND's own engine, compiled from its
// installed source header and driven through its public seed / subsequence /
// skip-ahead interface only.
//
// stdin: lines "seed stream node block" (decimal).  The engine is seeded
// with `seed` (key = low and high words of the seed), skips `stream`
// subsequences (counter words 2 and 3) and then 4 * (node + block * 2^32)
// numbers (counter words 0 and 1; the block part in four skips of
// block * 2^32 numbers each, so no skip overflows 64 bits), so it stands at
// counter (node, block, stream, 0); stdout: the four output words of that
// counter.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

int main() {
    unsigned long long seed, stream, node, block;
    while (std::scanf("%llu %llu %llu %llu", &seed, &stream, &node, &block) == 4) {
        rocrand_device::philox4x32_10_engine e(seed, stream, 0);
        e.discard(4ull * node);
        for (int i = 0; i < 4; ++i) e.discard(block << 32);
        const uint4 r = e.next4();
        std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
