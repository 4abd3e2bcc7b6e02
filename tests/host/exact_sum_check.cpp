// Host driver for the library's exact-sum code (csrc/exact_sum.h), built by
// tests/test_exact_sum_host.py with g++ and the address and undefined-behaviour
// sanitizers.  Each input line is "mbits n b_1 .. b_n": the float32 bit
// patterns (hex) of n values whose significands have mbits explicit bits.
// Each output line is "<rounded> <cheap> <forward> <backward>": the
// accumulator's rounded sum as float64 bits (hex), whether exact_by_range
// holds for the values' magnitude keys (0/1), and the plain float64 sums in
// forward and backward order (hex).
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "exact_sum.h"

static uint64_t bits_of(double x) {
  uint64_t b;
  std::memcpy(&b, &x, sizeof b);
  return b;
}

static double value_of(uint32_t b) {
  float f;
  std::memcpy(&f, &b, sizeof f);
  return (double)f;
}

int main() {
  int mbits;
  long long n;
  while (std::scanf("%d %lld", &mbits, &n) == 2) {
    std::vector<uint32_t> v((size_t)n);
    for (long long i = 0; i < n; ++i) std::scanf("%x", &v[(size_t)i]);
    fsa_exact::ExactSum acc;
    acc.clear();
    uint32_t kmin = fsa_exact::kKeyMinInit, kmax = fsa_exact::kKeyMaxInit;
    double fwd = 0.0, bwd = 0.0;
    for (long long i = 0; i < n; ++i) {
      const uint32_t b = v[(size_t)i];
      acc.add(b);
      const uint32_t a = b & 0x7FFFFFFFu;
      kmin = a - 1u < kmin ? a - 1u : kmin;
      kmax = a > kmax ? a : kmax;
      fwd = fwd + value_of(b);
      bwd = bwd + value_of(v[(size_t)(n - 1 - i)]);
    }
    // half of the values through a second accumulator, merged: the same sum
    fsa_exact::ExactSum a1, a2;
    a1.clear();
    a2.clear();
    for (long long i = 0; i < n; ++i) (i % 2 ? a1 : a2).add(v[(size_t)i]);
    a1.merge(a2);
    const double r = acc.rounded();
    if (bits_of(a1.rounded()) != bits_of(r) && r == r) return 3;
    std::printf("%016llx %d %016llx %016llx\n", (unsigned long long)bits_of(r),
                fsa_exact::exact_by_range(kmin, kmax, n, mbits) ? 1 : 0,
                (unsigned long long)bits_of(fwd + 0.0), (unsigned long long)bits_of(bwd + 0.0));
  }
  return 0;
}
