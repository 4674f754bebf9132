// msa_select.hpp -- exact wave-level top-m selection without exponentials or sorting.
//
// Block selection ("MiniMax-M3: MSA 技术报告速读", section 核心机制, the TopK equation and the
// forced local block) needs, per (query row, group), the best m blocks under the order
// (score desc, block index asc). Scores become order-preserving uint32 keys (key 0 marks an
// empty slot) and a wave holding V items per lane finds the exact m-th item by
//   1. a ballot-counted bitwise search over the 64 lane maxima (a lower bound on the
//      threshold that at least m items reach),
//   2. ranking only the items at or above that bound (normally a few dozen) in LDS,
//   3. an exact bitwise search over all items when ties make that set too large.
#pragma once

#include "msa_device.hpp"

namespace msa {

constexpr int SELECT_CAP = 256;  // candidates ranked in LDS (4 per lane)

__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Exact m-th item (1 <= m <= 63) of the wave's items under (key desc, idx asc); at least m
// slots are non-empty. lk / li: wave-private LDS of SELECT_CAP + 1 entries. On return, an
// item is among the best m iff key > kstar || (key == kstar && idx <= istar).
template <int V>
__device__ void wave_threshold(const uint32_t (&key)[V], const int32_t (&idx)[V], int m,
                               uint32_t *lk, int32_t *li, uint32_t &kstar, int32_t &istar) {
  constexpr int CAP = SELECT_CAP;
  const int lane = lane_id();
  uint32_t lm = 0;
#pragma unroll
  for (int s = 0; s < V; ++s) lm = max(lm, key[s]);
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = T | (1u << bit);
    if (popc64(ballot(lm >= c)) >= m) T = c;
  }
  T = max(T, 1u);
  int C = 0;
#pragma unroll
  for (int s = 0; s < V; ++s) C += popc64(ballot(key[s] >= T));

  if (C <= CAP) {
    int base = 0;
#pragma unroll
    for (int s = 0; s < V; ++s) {
      const bool pr = key[s] >= T;
      const uint64_t mk = ballot(pr);
      if (pr) {
        const int pos = base + rank_below(mk);
        lk[pos] = key[s];
        li[pos] = idx[s];
      }
      base += popc64(mk);
    }
    lds_wait();
    uint32_t ck[CAP / 64];
    int32_t ci[CAP / 64];
    int rk[CAP / 64];
#pragma unroll
    for (int q = 0; q < CAP / 64; ++q) {
      const int j = lane + 64 * q;
      ck[q] = j < C ? lk[j] : 0u;
      ci[q] = j < C ? li[j] : 0x7fffffff;
      rk[q] = 0;
    }
    for (int x = 0; x < C; ++x) {
      const uint32_t kx = lk[x];
      const int32_t ix = li[x];
#pragma unroll
      for (int q = 0; q < CAP / 64; ++q) rk[q] += (kx > ck[q]) || (kx == ck[q] && ix < ci[q]);
    }
    lds_wait();
#pragma unroll
    for (int q = 0; q < CAP / 64; ++q)
      if (lane + 64 * q < C && rk[q] == m - 1) {
        lk[CAP] = ck[q];
        li[CAP] = ci[q];
      }
    lds_wait();
    kstar = lk[CAP];
    istar = li[CAP];
    lds_wait();
    return;
  }
  // Heavy ties: exact search over every item.
  T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = T | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int s = 0; s < V; ++s) cnt += popc64(ballot(key[s] >= c));
    if (cnt >= m) T = c;
  }
  int ngt = 0;
#pragma unroll
  for (int s = 0; s < V; ++s) ngt += popc64(ballot(key[s] > T));
  const int need = m - ngt;  // >= 1 items with key == T are taken, lowest indices first
  int32_t X = 0;
  for (int bit = 30; bit >= 0; --bit) {
    const int32_t c = X | (1 << bit);
    int cnt = 0;
#pragma unroll
    for (int s = 0; s < V; ++s) cnt += popc64(ballot(key[s] == T && idx[s] < c));
    if (cnt < need) X = c;
  }
  kstar = T;
  istar = X;
}

__device__ __forceinline__ bool taken(uint32_t k, int32_t i, uint32_t ks, int32_t is) {
  return k != 0u && (k > ks || (k == ks && i <= is));
}

}  // namespace msa
