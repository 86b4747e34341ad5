// Independent reference for the oracle's noise stream: rocRAND's host-callable
// Philox4x32-10 engine (MIT-licensed source header shipped with ROCm).
// Usage: rocrand_philox_ref SEED SUBSEQUENCE OFFSET COUNT
// Prints COUNT 32-bit words, one per line, starting at stream element OFFSET.
#include <cstdio>
#include <cstdlib>
#include <rocrand/rocrand_philox4x32_10.h>

int main(int argc, char** argv) {
    if (argc != 5) { std::fprintf(stderr, "usage: seed subsequence offset count\n"); return 2; }
    unsigned long long seed = std::strtoull(argv[1], nullptr, 0);
    unsigned long long sub = std::strtoull(argv[2], nullptr, 0);
    unsigned long long off = std::strtoull(argv[3], nullptr, 0);
    long long count = std::strtoll(argv[4], nullptr, 0);
    rocrand_device::philox4x32_10_engine eng(seed, sub, off);
    for (long long i = 0; i < count; ++i) std::printf("%u\n", eng.next());
    return 0;
}
