// Known-answer helper for the oracle's Philox4x32-10: runs rocRAND's own
// implementation of the 10-round bijection (an independent implementation of
// Salmon et al., SC'11) on counters read from stdin.  Host-only; built and run
// by tests/test_oracle_pins.py.  Input lines: "c0 c1 c2 c3 k0 k1"; output
// lines: the four output words.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

namespace {
struct RawPhilox : rocrand_device::philox4x32_10_engine {
    uint4 apply(uint4 ctr, uint2 key) { return this->ten_rounds(ctr, key); }
};
}  // namespace

int main()
{
    unsigned c0, c1, c2, c3, k0, k1;
    RawPhilox engine;
    while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        uint4 r = engine.apply(uint4{c0, c1, c2, c3}, uint2{k0, k1});
        std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
