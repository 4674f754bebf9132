// msa_select.hpp -- exact wave-level top-m selection without exponentials or sorting.
//
// Block selection ("MiniMax-M3: MSA 技术报告速读", section 核心机制, the TopK equation and the
// forced local block) needs, per (query row, group), the best m blocks under the order
// (score desc, block index asc). Scores become order-preserving uint32 keys (key 0 marks an
// empty slot) and a wave holding V items per lane finds the exact m-th item by
//   1. a ballot-counted bitwise search over the 64 lane maxima (a lower bound on the
//      threshold that at least m items reach),
//   2. compacting the items at or above that bound (normally a few dozen) into LDS and
//      finding the exact m-th among them: by ranking every candidate against the others
//      when there are at most 64, else by a second bitwise search (keys, then indices for
//      ties at the threshold),
//   3. an exact bitwise search over all items when ties make that set too large.
#pragma once

#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {

constexpr int SELECT_CAP = 256;  // candidates ranked in LDS (4 per lane)
constexpr int SELECT_LDS = SELECT_CAP + 64;  // entries of a wave's lk / li: CAP + a spare per lane

__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// The m-th largest of N keys per lane (over the wave), given lo <= it <= hi: the bits
// above the highest bit where lo and hi differ are fixed, the rest come from a
// ballot-counted bitwise search (none at all when lo == hi, as under heavy ties).
template <int N>
__device__ __forceinline__ uint32_t mth_key(const uint32_t (&k)[N], int m, uint32_t lo, uint32_t hi) {
  const uint32_t diff = lo ^ hi;
  if (!diff) return lo;
  const int top = 31 - __builtin_clz(diff);
  uint32_t K = top == 31 ? 0u : lo & ~((2u << top) - 1u);
  for (int bit = top; bit >= 0; --bit) {
    const uint32_t c = K | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < N; ++q) cnt += popc64(ballot(k[q] >= c));
    if (cnt >= m) K = c;
  }
  return K;
}

// Item indices first + 64 s in slot s (a run of consecutive blocks, one per lane and slot),
// computed where they are used instead of being held in V registers per lane. Anything
// indexable by slot serves as the index argument below: such a run or an array.
struct StridedIdx {
  int32_t first;  // this lane's index in slot 0
  __device__ __forceinline__ int32_t operator[](int s) const { return first + 64 * s; }
};

// The index of the need-th (1-based) item with key K, counting in item order (slot-major,
// then lane), which is ascending index order: the cut among the items tied at K.
template <int N, typename IX>
__device__ __forceinline__ int32_t tie_cut(const uint32_t (&k)[N], const IX &ix, uint32_t K,
                                           int need) {
  int seen = 0;
  int32_t X = 0x7fffffff;
#pragma unroll
  for (int q = 0; q < N; ++q) {
    const bool eq = k[q] == K;
    const uint64_t mk = ballot(eq);
    const int c = popc64(mk);
    if (seen < need && seen + c >= need) {  // wave-uniform: the cut lies in this slot
      const uint64_t hit = ballot(eq && rank_below(mk) == need - seen - 1);
      X = __builtin_amdgcn_readlane(ix[q], __builtin_ctzll(hit));
    }
    seen += c;
  }
  return X;
}

// Exact m-th item (1 <= m <= 63) of the wave's items under (key desc, idx asc); at least m
// slots are non-empty, the non-empty items have distinct indices, and item order (slot-major,
// then lane) is ascending index order among the non-empty items (every caller's items are
// blocks in ascending order, or winners kept in that order). lk / li: wave-private LDS of
// SELECT_LDS entries (the last 64 are write-only spares, one per lane). On return, an
// item is among the best m iff key > kstar || (key == kstar && idx <= istar).
// Returns C >= m when the items with key >= a lower bound T (C of them, in item order:
// slot-major, then lane) are left in lk / li, or -1 when heavy ties sent it to the
// exhaustive search (lk / li then hold nothing useful).
template <int V, typename IX>
__device__ int wave_threshold(const uint32_t (&key)[V], const IX &idx, int m,
                              uint32_t *lk, int32_t *li, uint32_t &kstar, int32_t &istar) {
  constexpr int CAP = SELECT_CAP;
  constexpr int Q = CAP / 64;
  uint32_t lm = 0;
#pragma unroll
  for (int s = 0; s < V; ++s) lm = max(lm, key[s]);
  // Largest T that at least m lane maxima reach: at least m items are >= T.
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = T | (1u << bit);
    if (popc64(ballot(lm >= c)) >= m) T = c;
  }
  T = max(T, 1u);
  // Compact the items >= T into LDS in item order. A slot with none is skipped (a uniform
  // branch; usually about a quarter of them); otherwise every lane writes (no divergent
  // branch): items below T, and positions past CAP, go to the lane's own spare slot.
  int C = 0;
  const int spare = CAP + lane_id();
#pragma unroll
  for (int s = 0; s < V; ++s) {
    const bool pr = key[s] >= T;
    const uint64_t mk = ballot(pr);
    if (mk) {
      const int at = C + rank_below(mk);
      const int pos = (pr && at < CAP) ? at : spare;
      lk[pos] = key[s];
      li[pos] = idx[s];
      C += popc64(mk);
    }
  }
  if (C <= 64) {
    // Few candidates (the usual case): rank each one against all of them. Indices are
    // distinct, so (key desc, idx asc) orders the candidates totally, their ranks are
    // 0 .. C-1, and the candidate of rank m-1 is the m-th item.
    if (lane_id() < 4) lk[C + lane_id()] = 0u;  // padding for the 4-wide loop: ranks last
    lds_wait();
    const bool mine = lane_id() < C;
    const uint32_t k0 = mine ? lk[lane_id()] : 0u;
    const int32_t i0 = mine ? li[lane_id()] : 0;
    const uint64_t c0 = ((uint64_t)k0 << 32) | (0x7fffffffu - (uint32_t)i0);
    int rank = 0;
    for (int j = 0; j < C; j += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint64_t cj = ((uint64_t)lk[j + u] << 32) | (0x7fffffffu - (uint32_t)li[j + u]);
        rank += cj > c0 ? 1 : 0;
      }
    }
    const uint64_t hit = ballot(mine && rank == m - 1);
    if (hit) {  // always, for distinct indices
      const int src = __builtin_ctzll(hit);
      kstar = (uint32_t)__builtin_amdgcn_readlane((int)k0, src);
      istar = __builtin_amdgcn_readlane(i0, src);
      return C;
    }
  }
  if (C <= CAP) {
    lds_wait();
    // Empty slots hold key 0, which no search step below counts (every probe is >= 1).
    uint32_t ck[Q];
    int32_t ci[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int j = lane_id() + 64 * q;
      ck[q] = j < C ? lk[j] : 0u;
      ci[q] = j < C ? li[j] : 0x7fffffff;
    }
    // The m-th largest candidate key K (between T and the largest key), then the index
    // cut among the candidates tied at K: they sit in item order, so the `need` lowest
    // indices are the first `need` of them.
    const uint32_t K = mth_key(ck, m, T, wave_max_u32(lm));
    int ngt = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q) ngt += popc64(ballot(ck[q] > K));
    kstar = K;
    istar = tie_cut(ck, ci, K, m - ngt);  // 1 <= m - ngt <= the number tied at K
    return C;
  }
  // Heavy ties: the same over every item (T is still a lower bound of the m-th key).
  const uint32_t K = mth_key(key, m, T, wave_max_u32(lm));
  int ngt = 0;
#pragma unroll
  for (int s = 0; s < V; ++s) ngt += popc64(ballot(key[s] > K));
  kstar = K;
  istar = tie_cut(key, idx, K, m - ngt);
  return -1;
}

__device__ __forceinline__ bool taken(uint32_t k, int32_t i, uint32_t ks, int32_t is) {
  return k != 0u && (k > ks || (k == ks && i <= is));
}

// Final merge of one problem whose candidates are the winners of its key ranges (total
// pairs ck / ci, at most TOPK_CHUNK, in ascending block order), by NW waves of a workgroup.
// Stage 1 (every wave): wave w keeps the best m of its share, in item order, as entries
// [w * m, (w + 1) * m) of w_key / w_idx (NW * 64 entries), padded with key 0. lk / li: the
// wave's own SELECT_LDS entries of scratch.
template <int NW>
__device__ __forceinline__ void wide_stage1(const uint32_t *ck, const int32_t *ci, int total,
                                            int m, int w, uint32_t *lk, int32_t *li,
                                            uint32_t *w_key, int32_t *w_idx) {
  constexpr int NV = TOPK_CHUNK / (64 * NW);  // candidates per lane
  const int lane = lane_id();
  uint32_t key[NV];
  int32_t idx[NV];
  int nv = 0;
#pragma unroll
  for (int s = 0; s < NV; ++s) {
    const int ec = min((w * NV + s) * 64 + lane, total - 1);  // unconditional loads
    key[s] = ck[ec];
    idx[s] = ci[ec];
  }
#pragma unroll
  for (int s = 0; s < NV; ++s) {
    pin(key[s]);
    pin(idx[s]);
  }
#pragma unroll
  for (int s = 0; s < NV; ++s) {
    const bool in = (w * NV + s) * 64 + lane < total;
    key[s] = in ? key[s] : 0u;
    idx[s] = in ? idx[s] : 0x7fffffff;
    nv += popc64(ballot(key[s] != 0u));
  }
  uint32_t ks = 0;
  int32_t is = 0x7fffffff;
  if (nv > m) wave_threshold(key, idx, m, lk, li, ks, is);
  int pos = 0;
#pragma unroll
  for (int s = 0; s < NV; ++s) {
    const bool pr = taken(key[s], idx[s], ks, is);
    const uint64_t mk = ballot(pr);
    if (pr) {
      w_key[w * m + pos + rank_below(mk)] = key[s];
      w_idx[w * m + pos + rank_below(mk)] = idx[s];
    }
    pos += popc64(mk);
  }
  if (lane >= pos && lane < m) {
    w_key[w * m + lane] = 0u;
    w_idx[w * m + lane] = 0x7fffffff;
  }
}

// Stage 2 (one wave, after the workgroup has synchronised on stage 1): the best m of the
// NW * m entries, entry j in lane j % 64 (packed this way the winners spread over all
// lanes, which keeps the lane-maximum bound of the selection tight; a wave-per-slot layout
// leaves them on m lanes, and the bound admits nearly all). The waves' winners arrive in
// ascending block order and each wave kept its own in that order, so the winners come out
// in ascending block order: put(j, block) for j = 0 .. m-1.
template <int NW, typename Put>
__device__ __forceinline__ void wide_stage2(int m, const uint32_t *w_key, const int32_t *w_idx,
                                            uint32_t *lk, int32_t *li, Put put) {
  const int lane = lane_id();
  uint32_t k2[NW];
  int32_t i2[NW];
#pragma unroll
  for (int s = 0; s < NW; ++s) {
    const int j = s * 64 + lane;
    k2[s] = j < NW * m ? w_key[j] : 0u;
    i2[s] = j < NW * m ? w_idx[j] : 0x7fffffff;
  }
  uint32_t ks = 0;
  int32_t is = 0x7fffffff;
  wave_threshold(k2, i2, m, lk, li, ks, is);
  int pos = 0;
#pragma unroll
  for (int s = 0; s < NW; ++s) {
    const bool pr = taken(k2[s], i2[s], ks, is);
    const uint64_t mk = ballot(pr);
    if (pr) put(pos + rank_below(mk), i2[s]);
    pos += popc64(mk);
  }
}

}  // namespace msa
