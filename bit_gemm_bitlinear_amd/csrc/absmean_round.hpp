// Exact mean of |w| from per-exponent significand sums, rounded once to fp32.
//
// Part of the weight scale of the Falcon-Edge blog's _weight_quant ("A series
// of powerful, universal and fine-tunable 1.58-bit language models", section
// "Falcon-Edge, a series of universal models"): mean|w| is taken as the exact
// real sum divided by the element count, rounded to the nearest fp32 (ties to
// even, subnormals included), so it does not depend on summation order.
//
// buckets[E] holds the sum of the 24-bit significands of every |w| whose
// biased exponent is E (|w| = m * 2^(max(E,1) - 150)).  Plain C++ so the same
// code runs in the single-thread finalize kernel and in host-side checks.
#pragma once

#include <stdint.h>
#include <string.h>

#if defined(__HIPCC__)
#define BL_HD __host__ __device__
#else
#define BL_HD
#endif

namespace bl {

BL_HD inline uint32_t absmean_bits_from_buckets(const unsigned long long* buckets,
                                                uint64_t count) {
  constexpr int kLimbs = 14;  // 448 bits: 253-bit shift + 64-bit bucket + carries
  uint32_t limb[kLimbs];
  for (int i = 0; i < kLimbs; ++i) limb[i] = 0u;
  for (int e = 0; e < 255; ++e) {
    unsigned long long v = buckets[e];
    if (!v) continue;
    int sh = (e > 0 ? e : 1) - 1;  // total is kept in units of 2^-149
    int li = sh >> 5, bo = sh & 31;
    uint32_t parts[3];  // v << bo spans three 32-bit words
    parts[0] = (uint32_t)(v << bo);
    parts[1] = bo ? (uint32_t)(v >> (32 - bo)) : (uint32_t)(v >> 32);
    parts[2] = bo ? (uint32_t)(v >> (64 - bo)) : 0u;
    uint64_t carry = 0;
    for (int j = li; j < kLimbs; ++j) {
      uint64_t add = (j - li < 3) ? parts[j - li] : 0u;
      uint64_t t = (uint64_t)limb[j] + add + carry;
      limb[j] = (uint32_t)t;
      carry = t >> 32;
      if (j - li >= 2 && carry == 0) break;
    }
  }
  int top_bit = -1;
  for (int j = kLimbs - 1; j >= 0 && top_bit < 0; --j)
    if (limb[j]) top_bit = 32 * j + 31 - __builtin_clz(limb[j]);
  if (top_bit < 0) return 0u;

  // Q = floor(total * 2^S / count) by bit-serial long division.  With
  // count < 2^40 and total >= 1, Q >= 2^26: its 26 leading bits plus a
  // sticky bit (any lower quotient bit or a non-zero remainder) decide the
  // rounding.
  constexpr int S = 66;
  uint64_t r = 0, top26 = 0;
  int lq = 0;
  bool sticky = false;
  for (int b = top_bit + S; b >= 0; --b) {
    uint32_t bit = 0;
    if (b >= S) {
      int t = b - S;
      bit = (limb[t >> 5] >> (t & 31)) & 1u;
    }
    r = (r << 1) | bit;
    uint32_t qb = 0;
    if (r >= count) {
      r -= count;
      qb = 1;
    }
    if (lq == 0 && !qb) continue;
    ++lq;
    if (lq <= 26)
      top26 = (top26 << 1) | qb;
    else
      sticky = sticky || (qb != 0);
  }
  sticky = sticky || (r != 0);

  // value = Q * 2^(-149 - S); its leading bit has weight 2^e.  fp32 keeps 24
  // bits for normal values and down to 2^-149 for subnormal ones.
  const int e = (lq - 1) - 149 - S;
  const int keep = (e + 150 < 24) ? (e + 150) : 24;
  const int drop = 26 - keep;  // >= 2
  if (drop > 26) return 0u;    // below half the smallest subnormal
  uint64_t mant = top26 >> drop;
  const uint64_t guard = (top26 >> (drop - 1)) & 1u;
  const bool rest = sticky || ((top26 & ((1ull << (drop - 1)) - 1ull)) != 0);
  if (guard && (rest || (mant & 1u))) ++mant;
  if (e >= -126) return (uint32_t)(((uint64_t)(e + 127) << 23) + mant - (1ull << 23));
  return (uint32_t)mant;  // a carry to 2^23 lands on the smallest normal
}

}  // namespace bl
