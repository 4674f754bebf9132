// msa_topk.hip -- per-(query row, group) block selection.
//
// Definition ("MiniMax-M3: MSA 技术报告速读", section 核心机制: the TopK equation over block
// scores, and the rule that the query's own block is always selected): sel = the local
// block plus the top_k-1 earlier blocks with the highest block score; equal scores go to
// the lower block index; a row that sees top_k blocks or fewer selects them all; output
// ascending, -1 padded.
//
// No exponentials and no sort: scores become order-preserving uint32 keys, and a wave
// finds the exact (top_k-1)-th item of the total order (key desc, index asc) by
//   1. a ballot-counted bitwise search over the 64 lane maxima (a lower bound on the
//      threshold: at least m items reach it),
//   2. ranking only the items at or above that bound (normally a few dozen) in LDS,
//   3. an exact bitwise search over all items when ties make that set too large.
// Problems with more than TOPK_CHUNK candidate blocks are cut into chunks whose best
// top_k-1 are merged by a second pass with the same routine.
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {
namespace {

constexpr int V = TOPK_CHUNK / 64;  // items per lane
constexpr int CAP = 256;            // candidates ranked in LDS (4 per lane)

__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Exact m-th item (1 <= m <= 63) of the wave's items under (key desc, idx asc); key 0 is an
// empty slot and at least m slots are non-empty. On return, an item is among the best m
// iff key > kstar || (key == kstar && idx <= istar).
__device__ void wave_threshold(const uint32_t (&key)[V], const int32_t (&idx)[V], int m,
                               uint32_t *lk, int32_t *li, uint32_t &kstar, int32_t &istar) {
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

// Pass 1. Grid: x = groups of 4 problems (one wave each), y = chunk.
__global__ __launch_bounds__(256) void topk_pass1(TopkArgs a) {
  __shared__ uint32_t s_key[4][CAP + 1];
  __shared__ int32_t s_idx[4][CAP + 1];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long n_prob = (long)a.batch * a.h_kv * a.n_q;
  const long pid = (long)blockIdx.x * 4 + w;
  if (pid >= n_prob) return;
  const int chunk = blockIdx.y;
  const int t = (int)(pid % a.n_q);
  const long p = (long)a.q_start + t;
  const int local = (int)(p / a.block_size);
  const int k = a.top_k, m = k - 1;
  int32_t *out = a.sel + pid * k;
  if (local + 1 <= k) {  // sees k blocks or fewer: all of them
    if (chunk == 0 && lane < k) out[lane] = lane <= local ? lane : -1;
    return;
  }
  if (m == 0) {  // top_k == 1: the local block alone
    if (chunk == 0 && lane == 0) out[0] = local;
    return;
  }
  const int n_c = local;  // candidates: blocks 0 .. local-1
  const int nch = (n_c + TOPK_CHUNK - 1) / TOPK_CHUNK;
  if (chunk >= nch) return;
  const int base = chunk * TOPK_CHUNK;
  const float *row = a.bmax + pid * (long)a.n_blocks;
  uint32_t key[V];
  int32_t idx[V];
#pragma unroll
  for (int s = 0; s < V; ++s) {
    const int c = base + s * 64 + lane;
    idx[s] = c;
    key[s] = c < n_c ? order_key(row[c]) : 0u;
  }
  const int valid = min(TOPK_CHUNK, n_c - base);
  if (nch == 1) {
    uint32_t ks;
    int32_t is;
    wave_threshold(key, idx, m, s_key[w], s_idx[w], ks, is);
    int pos = 0;
#pragma unroll
    for (int s = 0; s < V; ++s) {  // slot-major order is ascending block order
      const bool pr = taken(key[s], idx[s], ks, is);
      const uint64_t mk = ballot(pr);
      if (pr) out[pos + rank_below(mk)] = idx[s];
      pos += popc64(mk);
    }
    if (lane == 0) out[m] = local;
    return;
  }
  uint32_t *ck = a.cand_key + (pid * a.n_chunks + chunk) * (long)m;
  int32_t *ci = a.cand_idx + (pid * a.n_chunks + chunk) * (long)m;
  uint32_t ks = 0;
  int32_t is = 0x7fffffff;
  if (valid > m) wave_threshold(key, idx, m, s_key[w], s_idx[w], ks, is);
  int pos = 0;
#pragma unroll
  for (int s = 0; s < V; ++s) {
    const bool pr = taken(key[s], idx[s], ks, is);
    const uint64_t mk = ballot(pr);
    if (pr) {
      ck[pos + rank_below(mk)] = key[s];
      ci[pos + rank_below(mk)] = idx[s];
    }
    pos += popc64(mk);
  }
  if (lane >= pos && lane < m) {  // a short last chunk leaves empty slots
    ck[lane] = 0u;
    ci[lane] = -1;
  }
}

// Pass 2: merge the chunk winners of problems with more than one chunk. One wave each.
__global__ __launch_bounds__(256) void topk_pass2(TopkArgs a) {
  __shared__ uint32_t s_key[4][CAP + 1];
  __shared__ int32_t s_idx[4][CAP + 1];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long n_prob = (long)a.batch * a.h_kv * a.n_q;
  const long pid = (long)blockIdx.x * 4 + w;
  if (pid >= n_prob) return;
  const int t = (int)(pid % a.n_q);
  const long p = (long)a.q_start + t;
  const int local = (int)(p / a.block_size);
  const int k = a.top_k, m = k - 1;
  if (local + 1 <= k || m == 0) return;
  const int nch = (local + TOPK_CHUNK - 1) / TOPK_CHUNK;
  if (nch == 1) return;
  const int total = nch * m;  // <= TOPK_CHUNK (checked on the host)
  const uint32_t *ck = a.cand_key + pid * a.n_chunks * (long)m;
  const int32_t *ci = a.cand_idx + pid * a.n_chunks * (long)m;
  uint32_t key[V];
  int32_t idx[V];
#pragma unroll
  for (int s = 0; s < V; ++s) {
    const int e = s * 64 + lane;
    key[s] = e < total ? ck[e] : 0u;
    idx[s] = e < total ? ci[e] : 0x7fffffff;
  }
  uint32_t ks;
  int32_t is;
  wave_threshold(key, idx, m, s_key[w], s_idx[w], ks, is);
  // Collect the m winners, then place each by its rank in block order.
  uint32_t *list = reinterpret_cast<uint32_t *>(s_idx[w]);
  int pos = 0;
#pragma unroll
  for (int s = 0; s < V; ++s) {
    const bool pr = taken(key[s], idx[s], ks, is);
    const uint64_t mk = ballot(pr);
    if (pr) list[pos + rank_below(mk)] = (uint32_t)idx[s];
    pos += popc64(mk);
  }
  lds_wait();
  int32_t *out = a.sel + pid * k;
  if (lane < m) {
    const uint32_t mine = list[lane];
    int rank = 0;
    for (int x = 0; x < m; ++x) rank += list[x] < mine;
    out[rank] = (int32_t)mine;
  }
  if (lane == 0) out[m] = local;
}

}  // namespace

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
  const long n_prob = (long)a.batch * a.h_kv * a.n_q;
  const unsigned groups = (unsigned)((n_prob + 3) / 4);
  hipLaunchKernelGGL(topk_pass1, dim3(groups, (unsigned)a.n_chunks), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_chunks <= 1) return e;
  hipLaunchKernelGGL(topk_pass2, dim3(groups), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace msa
