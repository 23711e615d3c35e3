// Per-block top-n selection (host and device).
//
// Rule (guide s2.1, N:M: keep n of every m consecutive channels): position j
// of an m-block is kept when fewer than n positions beat it, where q beats j
// if its score is larger, or equal with q < j.  Exactly n are kept.
//
// Scores are |x - eta| * f with f >= 0, i.e. non-negative floats whose bit
// patterns order like the values (+0 is the only zero that can occur).  The
// n-th largest score t is found by sorting the bit patterns with Batcher's
// odd-even merge network (min/max only); every score above t is kept, and
// of the scores equal to t the lowest positions fill the remaining places.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define SPA_HD __host__ __device__ __forceinline__
#else
#define SPA_HD inline
#endif

namespace spa {

template <class V>
SPA_HD V umin(V a, V b) { return a < b ? a : b; }
template <class V>
SPA_HD V umax(V a, V b) { return a < b ? b : a; }

// Batcher's odd-even merge sort, ascending, M a power of two.
template <int M>
SPA_HD void oem_sort(uint32_t (&v)[M]) {
#pragma unroll
  for (int p = 1; p < M; p <<= 1)
#pragma unroll
    for (int k = p; k >= 1; k >>= 1)
#pragma unroll
      for (int j = k % p; j + k < M; j += 2 * k)
#pragma unroll
        for (int i = 0; i < k; ++i)
          if (i + j + k < M && (i + j) / (2 * p) == (i + j + k) / (2 * p)) {
            const uint32_t lo = umin(v[i + j], v[i + j + k]);
            const uint32_t hi = umax(v[i + j], v[i + j + k]);
            v[i + j] = lo;
            v[i + j + k] = hi;
          }
}

// Keep bits (bit j = position j kept) of one block of non-negative scores,
// given as their IEEE-754 bit patterns.
template <int M>
SPA_HD uint32_t topn_keep_bits(const uint32_t (&s)[M], int n) {
  uint32_t v[M];
#pragma unroll
  for (int j = 0; j < M; ++j) v[j] = s[j];
  oem_sort<M>(v);
  const uint32_t t = v[M - n];  // the n-th largest score
  int above = 0;
#pragma unroll
  for (int j = 0; j < M; ++j) above += s[j] > t ? 1 : 0;
  const int need = n - above;   // places left for scores equal to t, lowest positions first
  int seen = 0;
  uint32_t keep = 0;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    const bool eq = s[j] == t;
    const bool k = (s[j] > t) || (eq && seen < need);
    keep |= (k ? 1u : 0u) << j;
    seen += eq ? 1 : 0;
  }
  return keep;
}

// Top 2 of one 4-block by score (ties to the lower channel) as a tournament:
// the winner of each pair, the better of the two winners, then the runner-up
// -- the first pair's loser or the second pair's winner when the first pair
// holds the best, else the first pair's winner or the second pair's loser.
// Every channel of the first pair precedes every channel of the second, so a
// tie across the pairs goes to the first.  Four comparisons where the rank
// count takes six, and no bit scan: returns the 2:4 position code
// lo | hi << 2 and the kept values v[lo], v[hi].
SPA_HD uint32_t top2of4(const float (&s)[4], const float* v, float& vlo, float& vhi) {
  const bool a = s[0] >= s[1];                           // channel 0 wins its pair
  const bool b = s[2] >= s[3];                           // channel 2 wins its pair
  const float wa = __builtin_fmaxf(s[0], s[1]), la = __builtin_fminf(s[0], s[1]);
  const float wb = __builtin_fmaxf(s[2], s[3]), lb = __builtin_fminf(s[2], s[3]);
  const bool c = wa >= wb;                               // the first pair holds the best
  const bool d = c ? la >= wb : wa >= lb;                // ... and the runner-up
  const bool same = c == d;                              // both kept entries from one pair
  const float va = a ? v[0] : v[1], vb = b ? v[2] : v[3];
  vlo = same ? (c ? v[0] : v[2]) : va;
  vhi = same ? (c ? v[1] : v[3]) : vb;
  return same ? (c ? 4u : 14u) : ((a ? 0u : 1u) | (b ? 8u : 12u));
}

}  // namespace spa
