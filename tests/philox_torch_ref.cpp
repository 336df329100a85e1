// Prints the first four 32-bit outputs of PyTorch's header-only Philox4x32-10
// engine (ATen/core/PhiloxRNGEngine.h) for each "seed subsequence offset"
// line on stdin.  The engine starts from counter (offset low, offset high,
// subsequence low, subsequence high) and key (seed low, seed high), so its
// first block is Philox4x32-10 of that counter: an implementation of the
// generator written independently of the oracle's, used to pin it.
#include <ATen/core/PhiloxRNGEngine.h>

#include <cstdio>

int main() {
  unsigned long long seed, sub, off;
  while (std::scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
    at::philox_engine e(seed, sub, off);
    const unsigned a = e(), b = e(), c = e(), d = e();
    std::printf("%u %u %u %u\n", a, b, c, d);
  }
  return 0;
}
