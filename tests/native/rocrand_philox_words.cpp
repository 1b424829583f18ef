// Prints Philox4x32-10 words from rocRAND's engine (host side, public API) for
// the (seed, step, row, token) tuples read from stdin, one per line.  The
// engine's counter is (offset/4 as a 64-bit value, subsequence as a 64-bit
// value) and its key is the 64-bit seed, so token i of row b under step s is
// word (i mod 4) at offset 4*((b << 32) | (i >> 2)) of subsequence s.
// Test-only: an independent implementation to pin the oracle's Philox.
#include <cstdio>
#include <cstdint>
#include <rocrand/rocrand_philox4x32_10.h>

int main()
{
    unsigned long long seed, step, row, token;
    while (std::scanf("%llu %llu %llu %llu", &seed, &step, &row, &token) == 4) {
        unsigned long long offset = 4ull * ((row << 32) | (token >> 2)) + (token & 3ull);
        rocrand_device::philox4x32_10_engine eng(seed, step, offset);
        std::printf("%u\n", eng.next());
    }
    return 0;
}
