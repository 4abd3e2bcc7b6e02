// Exact sums of float32 / bfloat16 values, rounded once to float64.
//
// Frame and block selection pool tokens into float64 sums (Light Forcing
// §2.2: query and key tokens compressed by mean pooling).  A sum is defined as
// the exact sum of its values rounded once to the nearest float64, ties to
// even, so it has no summation order.  Two tools give it:
//
//   exact_by_range  the cheap case.  Every value of a segment is an integer
//                   multiple of the unit in the last place of its smallest
//                   nonzero magnitude, and every partial sum is below n times
//                   its largest magnitude.  When those two bounds are at most
//                   53 bits apart, every partial sum in any order is a
//                   float64, so plain float64 additions are exact and give the
//                   exact sum whatever their order.
//   ExactSum        the general case: a fixed-point accumulator of 32-bit
//                   digits (held in int64 limbs with room for carries) for
//                   values scaled by 2^149, the weight of the smallest float32
//                   subnormal; rounding the final integer to float64 takes its
//                   top 64 bits and a sticky bit.
//
// The functions compile for the host as well (FSA_HD may be defined empty),
// so the same code is checked on the CPU against exact rational arithmetic.
#pragma once

#include <cmath>
#include <cstdint>

#ifndef FSA_HD
#define FSA_HD __host__ __device__
#endif

namespace fsa_exact {

// Bits of the explicit significand: 7 for bfloat16, 23 for float32.
constexpr int kBf16Bits = 7;
constexpr int kF32Bits = 23;

// Magnitude keys of a set of values, as float32 bit patterns without the
// sign: kmin = smallest nonzero |x| bits minus 1 (0xFFFFFFFF when every value
// is zero; computed as min over (|x| bits - 1) with unsigned wrap-around, so
// zeros drop out), kmax = largest |x| bits.
constexpr uint32_t kKeyMinInit = 0xFFFFFFFFu;
constexpr uint32_t kKeyMaxInit = 0u;

FSA_HD inline int ceil_log2(long long n) {
  int lg = 0;
  while ((1LL << lg) < n) ++lg;
  return lg;
}

// True when float64 additions of the n values described by the keys are exact
// in every order (see above).  mbits: kBf16Bits or kF32Bits.
FSA_HD inline bool exact_by_range(uint32_t kmin, uint32_t kmax, long long n, int mbits) {
  if (kmin == kKeyMinInit) return true;  // every value is zero
  int emin = (int)(((kmin + 1u) >> 23) & 0xFFu);
  if (emin == 0) emin = 1;  // subnormals share the unit of the smallest normal binade
  const int emax = (int)((kmax >> 23) & 0xFFu);
  // |partial| < n * 2^(emax - 126); every value is a multiple of
  // 2^(emin - 127 - mbits); a float64 holds such multiples below 2^53 units
  return emax - emin + ceil_log2(n) <= 52 - mbits;
}

// Fixed-point accumulator: value = sum_j limb[j] * 2^(32 j) * 2^-149.  A
// float32 value m * 2^(e-150) (m < 2^24) adds m << (sh % 32), sh = e - 1,
// split over digits sh/32 and sh/32 + 1, so each limb gains less than 2^32
// per value: 2^31 values fit.  Non-finite values are summed apart in float64
// (the result is then that float64 sum: inf or NaN).
struct ExactSum {
  static constexpr int kLimbs = 10;  // 320 bits >= 278 value bits + 31 carry bits + sign
  long long limb[kLimbs];
  double nonfinite;
  bool has_nonfinite;

  FSA_HD void clear() {
#pragma unroll
    for (int i = 0; i < kLimbs; ++i) limb[i] = 0;
    nonfinite = 0.0;
    has_nonfinite = false;
  }

  // Adds the float32 value with bit pattern `bits` (a bfloat16 value is its
  // 16 bits shifted up by 16).  The digit index is data-dependent; the limbs
  // are updated through selects so that they stay in registers on the GPU.
  FSA_HD void add(uint32_t bits) {
    const uint32_t e = (bits >> 23) & 0xFFu;
    uint32_t m = bits & 0x7FFFFFu;
    if (e == 0xFFu) {
      float f;
      __builtin_memcpy(&f, &bits, sizeof f);
      nonfinite += (double)f;
      has_nonfinite = true;
      return;
    }
    if (e == 0u && m == 0u) return;
    int sh = 0;
    if (e != 0u) {
      m |= 0x800000u;
      sh = (int)e - 1;
    }
    const unsigned long long v = (unsigned long long)m << (sh & 31);
    long long lo = (long long)(v & 0xFFFFFFFFull), hi = (long long)(v >> 32);
    if (bits >> 31) {
      lo = -lo;
      hi = -hi;
    }
    const int j = sh >> 5;
#pragma unroll
    for (int i = 0; i < kLimbs; ++i) {
      limb[i] += (i == j ? lo : 0LL);
      limb[i] += (i == j + 1 ? hi : 0LL);
    }
  }

  // Adds another accumulator (exact: limb-wise integer addition).
  FSA_HD void merge(const ExactSum &o) {
#pragma unroll
    for (int i = 0; i < kLimbs; ++i) limb[i] += o.limb[i];
    nonfinite += o.nonfinite;
    has_nonfinite = has_nonfinite || o.has_nonfinite;
  }

  // The exact sum rounded to the nearest float64, ties to even; +0 for zero.
  // Every limb index below is a compile-time constant (unrolled loops and
  // selects), so on the GPU the limbs stay in registers.
  FSA_HD double rounded() const {
    if (has_nonfinite) return nonfinite;
    long long d[kLimbs];
#pragma unroll
    for (int i = 0; i < kLimbs; ++i) d[i] = limb[i];
    // carries: digits 0..8 into [0, 2^32), the top limb keeps the sign
#pragma unroll
    for (int i = 0; i + 1 < kLimbs; ++i) {
      const long long c = d[i] >> 32;  // floor division by 2^32
      d[i] -= c * 4294967296LL;
      d[i + 1] += c;
    }
    const bool neg = d[kLimbs - 1] < 0;
    if (neg) {
#pragma unroll
      for (int i = 0; i < kLimbs; ++i) d[i] = -d[i];
#pragma unroll
      for (int i = 0; i + 1 < kLimbs; ++i) {
        const long long c = d[i] >> 32;
        d[i] -= c * 4294967296LL;
        d[i + 1] += c;
      }
    }
    int h = -1;
#pragma unroll
    for (int i = 0; i < kLimbs; ++i) h = d[i] != 0 ? i : h;
    if (h < 0) return 0.0;
    // the top 96 bits w0:w1:w2 (w0 != 0), then the top 64 with the leading one at bit 63
    unsigned long long w0 = 0, w1 = 0, w2 = 0;
    bool sticky = false;
#pragma unroll
    for (int i = 0; i < kLimbs; ++i) {
      const unsigned long long di = (unsigned long long)d[i];
      w0 = i == h ? di : w0;
      w1 = i == h - 1 ? di : w1;
      w2 = i == h - 2 ? di : w2;
      sticky = sticky || (i < h - 2 && di != 0);
    }
    const int lz = __builtin_clzll(w0) - 32;  // leading zeros of the 32-bit digit w0
    unsigned long long top = (w0 << (32 + lz)) | (w1 << lz);
    if (lz > 0) top |= w2 >> (32 - lz);
    const unsigned long long below = lz > 0 ? (w2 & ((1ull << (32 - lz)) - 1ull)) : w2;
    sticky = sticky || below != 0;
    // top counts units of 2^(32 (h - 2) + 32 - lz - 149); keep 53 bits
    unsigned long long mant = top >> 11;
    const unsigned long long rem = top & 0x7FFull;
    if (rem > 0x400ull || (rem == 0x400ull && (sticky || (mant & 1ull)))) ++mant;
    int ex = 32 * (h - 2) + 32 - lz - 149 + 11;
    if (mant == (1ull << 53)) {
      mant >>= 1;
      ++ex;
    }
    const double r = ldexp((double)mant, ex);
    return neg ? -r : r;
  }
};

}  // namespace fsa_exact
