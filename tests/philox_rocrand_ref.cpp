// Host program used only by the oracle's CPU tests: prints words of rocRAND's
// Philox4x32-10 engine (seed, subsequence, offset) so the oracle's own Philox
// can be compared with an implementation it shares no code with.
// Usage: philox_rocrand_ref SEED SUBSEQUENCE OFFSET COUNT
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
    if (argc != 5) return 2;
    const unsigned long long seed = std::strtoull(argv[1], nullptr, 0);
    const unsigned long long sub = std::strtoull(argv[2], nullptr, 0);
    const unsigned long long off = std::strtoull(argv[3], nullptr, 0);
    const long count = std::strtol(argv[4], nullptr, 0);
    rocrand_device::philox4x32_10_engine eng(seed, sub, off);
    for (long i = 0; i < count; ++i) std::printf("%u\n", eng.next());
    return 0;
}
