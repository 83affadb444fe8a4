// Reads "key ctr0 ctr1 ctr2 ctr3" lines (decimal) and prints the four
// Philox4x32-10 output words that rocRAND's host-callable engine produces for
// that key and counter.  Used only by the oracle's Philox pin test.
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
    unsigned long long key, c0, c1, c2, c3;
    while (std::scanf("%llu %llu %llu %llu %llu", &key, &c0, &c1, &c2, &c3) == 5) {
        // The engine's counter is (offset/4 as 64 bits, subsequence as 64 bits).
        unsigned long long sub = (c3 << 32) | c2;
        unsigned long long n = (c1 << 32) | c0;
        rocrand_device::philox4x32_10_engine e(key, sub, 0);
        while (n) {
            unsigned long long step = n > ((1ull << 62) - 1) ? ((1ull << 62) - 1) : n;
            e.discard(4ull * step);
            n -= step;
        }
        unsigned a = e(), b = e(), c = e(), d = e();
        std::printf("%u %u %u %u\n", a, b, c, d);
    }
    return 0;
}
