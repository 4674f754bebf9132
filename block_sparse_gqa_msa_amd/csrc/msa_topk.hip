// msa_topk.hip -- per-(query row, group) block selection.
//
// Definition ("MiniMax-M3: MSA 技术报告速读", section 核心机制: the TopK equation over block
// scores, and the rule that the query's own block is always selected): sel = the local
// block plus the top_k-1 earlier blocks with the highest block score; equal scores go to
// the lower block index; a row that sees top_k blocks or fewer selects them all; output
// ascending, -1 padded.
//
// No exponentials and no sort: see msa_select.hpp for the wave-level exact threshold.
// Items past the end load from a valid address and are then blanked; the loads of a batch are
// issued together and pinned (see pin()), since loads under branches go one at a time.
// Problems with more than TOPK_CHUNK candidate blocks are cut into chunks whose best
// top_k-1 are merged by a second pass with the same routine; or, given run keys from the
// index kernel, only the runs of blocks that can hold a winner are read (topk_runs).
#include "msa_device.hpp"
#include "msa_internal.hpp"
#include "msa_select.hpp"

namespace msa {
namespace {

constexpr int V = TOPK_CHUNK / 64;  // items per lane

// Best m of candidates [base, base + valid) of one problem's block scores, VI per lane.
template <int VI>
__device__ __forceinline__ void select_chunk(const TopkArgs &a, long pid, int chunk, int base,
                                             int n_c, int valid, bool single, int local,
                                             uint32_t *lk, int32_t *li) {
  const int lane = lane_id();
  const int m = a.top_k - 1;
  int32_t *out = a.sel + pid * a.top_k;
  const float *row = a.bmax + pid * (long)a.n_blocks;
  uint32_t key[VI];
  const StridedIdx idx{base + lane};  // item (s, lane) is block base + 64 s + lane
  float x[VI];
  // The row address is the wave's (scalar); each item adds a 32-bit offset, clamped to the
  // last candidate (items past it are blanked below). A row gets 16 or 32 items per lane
  // only with more than 8 * 64 or 16 * 64 candidates, so the first half of its slots is
  // always full: no clamp and no blanking there.
  constexpr int FULL = VI > 8 ? VI / 2 : 0;
  const unsigned char *rowb = reinterpret_cast<const unsigned char *>(row);
#pragma unroll
  for (int s = 0; s < VI; ++s)
    x[s] = __builtin_nontemporal_load(reinterpret_cast<const float *>(
        rowb + (uint32_t)(s < FULL ? idx[s] : min(idx[s], n_c - 1)) * 4u));
#pragma unroll
  for (int s = 0; s < VI; ++s) pin(x[s]);
#pragma unroll
  for (int s = 0; s < VI; ++s) key[s] = (s < FULL || idx[s] < n_c) ? order_key(x[s]) : 0u;
  uint32_t *ck = a.cand_key + (pid * a.n_chunks + chunk) * (long)m;
  int32_t *ci = a.cand_idx + (pid * a.n_chunks + chunk) * (long)m;
  // Write the winners in item order (= ascending block order): to sel for a single chunk,
  // else as this chunk's candidates.
  auto put = [&](int at, uint32_t kv, int32_t iv) {
    if (single) {
      out[at] = iv;
    } else {
      ck[at] = kv;
      ci[at] = iv;
    }
  };
  uint32_t ks = 0;
  int32_t is = 0x7fffffff;
  int C = -1;
  if (valid > m) C = wave_threshold(key, idx, m, lk, li, ks, is);
  int pos = 0;
  if (C >= 0) {  // the winners are among the C candidates left in LDS, in item order
    for (int q = 0; q * 64 < C; ++q) {
      const int j = q * 64 + lane;
      const uint32_t kv = j < C ? lk[j] : 0u;
      const int32_t iv = j < C ? li[j] : 0;
      const bool pr = taken(kv, iv, ks, is);
      const uint64_t mk = ballot(pr);
      if (pr) put(pos + rank_below(mk), kv, iv);
      pos += popc64(mk);
    }
  } else {
#pragma unroll
    for (int s = 0; s < VI; ++s) {  // slot-major order is ascending block order
      const bool pr = taken(key[s], idx[s], ks, is);
      const uint64_t mk = ballot(pr);
      if (pr) put(pos + rank_below(mk), key[s], idx[s]);
      pos += popc64(mk);
    }
  }
  if (single) {
    if (lane == 0) out[m] = local;
  } else if (lane >= pos && lane < m) {  // a short last chunk leaves empty slots
    ck[lane] = 0u;
    ci[lane] = -1;
  }
}

// Pass 1. Grid: x = groups of 4 problems (one wave each), y = chunk. A wave ranks one
// problem, so the loads' latency is hidden by other resident waves, and the register
// budget is held to WPE waves per SIMD (the unconstrained allocation took 106 VGPRs, four
// waves). Rows of one chunk (at most 2048 candidates, a mix of 8, 16 and 32 items per
// lane) run best at six (80 VGPRs; 0.615 -> 0.576 ms at 128K), rows of several full
// chunks (32 items per lane throughout) at five (96 VGPRs; 0.496 against 0.508 ms on the
// 1M-context chunk), with no spills either way.
template <int WPE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE))) void topk_pass1(TopkArgs a) {
  __shared__ uint32_t s_key[4][SELECT_LDS];
  __shared__ int32_t s_idx[4][SELECT_LDS];
  // The wave index is made scalar so that the problem and its row address are too.
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
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
  const int valid = min(TOPK_CHUNK, n_c - base);
  // Items per lane sized to this chunk's candidates (wave-uniform choice).
  if (valid <= 512)
    select_chunk<8>(a, pid, chunk, base, n_c, valid, nch == 1, local, s_key[w], s_idx[w]);
  else if (valid <= 1024)
    select_chunk<16>(a, pid, chunk, base, n_c, valid, nch == 1, local, s_key[w], s_idx[w]);
  else
    select_chunk<V>(a, pid, chunk, base, n_c, valid, nch == 1, local, s_key[w], s_idx[w]);
}

// The best m of the winners of a problem's nch chunks (written by select_chunk, in
// ascending block order, chunk after chunk, a short chunk padded with key 0) into sel,
// local block last. One wave. Item order is block order among the non-empty items, so
// ties break by item number; win (64 entries of LDS) takes the winners' item numbers, and
// only their blocks are read.
__device__ __forceinline__ void merge_winners(const TopkArgs &a, long pid, int nch, int local,
                                              uint32_t *lk, int32_t *li, int32_t *win) {
  const int lane = lane_id();
  const int m = a.top_k - 1;
  int32_t *out = a.sel + pid * a.top_k;
  const int total = nch * m;  // <= TOPK_CHUNK (checked on the host)
  const uint32_t *ck = a.cand_key + pid * a.n_chunks * (long)m;
  const int32_t *ci = a.cand_idx + pid * a.n_chunks * (long)m;
  const StridedIdx item{lane};
  uint32_t key[V];
#pragma unroll
  for (int s = 0; s < V; ++s) key[s] = ck[min(item[s], total - 1)];  // unconditional loads
#pragma unroll
  for (int s = 0; s < V; ++s) pin(key[s]);
#pragma unroll
  for (int s = 0; s < V; ++s) key[s] = item[s] < total ? key[s] : 0u;
  uint32_t ks = 0;
  int32_t is = 0x7fffffff;
  const int C = wave_threshold(key, item, m, lk, li, ks, is);
  int pos = 0;
  if (C >= 0) {
    for (int q = 0; q * 64 < C; ++q) {
      const int j = q * 64 + lane;
      const uint32_t kv = j < C ? lk[j] : 0u;
      const int32_t iv = j < C ? li[j] : 0;
      const bool pr = taken(kv, iv, ks, is);
      const uint64_t mk = ballot(pr);
      if (pr) win[pos + rank_below(mk)] = iv;
      pos += popc64(mk);
    }
  } else {
#pragma unroll
    for (int s = 0; s < V; ++s) {
      const bool pr = taken(key[s], item[s], ks, is);
      const uint64_t mk = ballot(pr);
      if (pr) win[pos + rank_below(mk)] = item[s];
      pos += popc64(mk);
    }
  }
  lds_wait();
  if (lane < m) out[lane] = ci[win[lane]];  // exactly m winners, in ascending order
  if (lane == 0) out[m] = local;
}

// Pass 2: merge the chunk winners of problems with more than one chunk. One wave each.
__global__ __launch_bounds__(256) void topk_pass2(TopkArgs a) {
  __shared__ uint32_t s_key[4][SELECT_LDS];
  __shared__ int32_t s_idx[4][SELECT_LDS];
  __shared__ int32_t s_win[4][64];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long n_prob = (long)a.batch * a.h_kv * a.n_q;
  const long pid = (long)blockIdx.x * 4 + w;
  if (pid >= n_prob) return;
  const int t = (int)(pid % a.n_q);
  const long p = (long)a.q_start + t;
  const int local = (int)(p / a.block_size);
  const int k = a.top_k, m = k - 1;
  int32_t *out = a.sel + pid * k;
  if (local + 1 <= k || m == 0) {  // handled by pass 1, unless this pass is the only one
    if (a.final_all) {
      if (local + 1 <= k) {
        if (lane < k) out[lane] = lane <= local ? lane : -1;
      } else if (lane == 0) {
        out[0] = local;
      }
    }
    return;
  }
  const int nch = (local + a.chunk_blocks - 1) / a.chunk_blocks;
  if (nch == 1 && !a.final_all) return;
  merge_winners(a, pid, nch, local, s_key[w], s_idx[w], s_win[w]);
}

// Candidates 0 .. n_c-1 of one problem, with run keys (the order key of each aligned run's
// largest block maximum). Let T be the m-th largest key of the nf runs that lie wholly
// before the local block: at least m runs have a key >= T, each holding a block with that
// key, and a run whose key is below T has every block below each of those, so none of its
// blocks is among the best m, ties included. The winners therefore lie in the runs whose
// key reaches T or in the tail after the last whole run: phase 1 finds those runs, phase
// 2 ranks their blocks and the tail's. Normally about m runs reach T: 2 KiB of run keys
// and about m cache lines of maxima per problem at 1M context, against 64 KiB for the
// whole row. (A NaN block maximum, which finite inputs cannot give, does not raise its
// run's key.)

// Phase 1: the nf runs' keys, VI per lane; the runs whose key reaches the m-th largest,
// in ascending order, go to runs[] (64 entries; more are counted, not stored).
template <int VI>
__device__ __forceinline__ int runs_at_bound(const uint32_t *rrow, int nf, int m, uint32_t *lk,
                                             int32_t *li, int32_t *runs) {
  const int lane = lane_id();
  const StridedIdx idx{lane};  // item (s, lane) is run 64 s + lane
  uint32_t key[VI];
#pragma unroll
  for (int s = 0; s < VI; ++s) key[s] = __builtin_nontemporal_load(rrow + min(idx[s], nf - 1));
#pragma unroll
  for (int s = 0; s < VI; ++s) pin(key[s]);
#pragma unroll
  for (int s = 0; s < VI; ++s) key[s] = idx[s] < nf ? key[s] : 0u;
  uint32_t ks = 0;
  int32_t is = 0x7fffffff;
  const int C = wave_threshold(key, idx, m, lk, li, ks, is);
  int cnt = 0;
  auto keep = [&](bool pr, int32_t r) {  // in item order, which is ascending run order
    const uint64_t mk = ballot(pr);
    const int at = cnt + rank_below(mk);
    if (pr && at < 64) runs[at] = r;
    cnt += popc64(mk);
  };
  if (C >= 0) {  // every run at or above the bound is among the C left in LDS
    for (int q = 0; q * 64 < C; ++q) {
      const int j = q * 64 + lane;
      const uint32_t kv = j < C ? lk[j] : 0u;
      const int32_t iv = j < C ? li[j] : 0;
      keep(kv >= ks, iv);  // ks >= 1: padding (key 0) is never kept
    }
  } else {
#pragma unroll
    for (int s = 0; s < VI; ++s) keep(key[s] >= ks, idx[s]);
  }
  return cnt;
}

// Phase 2: rank the blocks of runs[0 .. nr) (cnt whole runs, then the tail of tcount
// blocks as run nf when tcount > 0), half a wave per run and slot; winners to sel in
// ascending block order, local block last. Item j = 64 s + lane is block j % 32 of run
// runs[j / 32]; the runs ascend, so item order is block order and the ranking can break
// ties by item number, which needs no register per item: only winners are turned into
// blocks.
template <int VI>
__device__ __forceinline__ void rank_runs(const TopkArgs &a, long pid, int local,
                                          const int32_t *runs, int cnt, int nr, int tcount,
                                          uint32_t *lk, int32_t *li) {
  const int lane = lane_id(), half = lane >> 5, sub = lane & (RUN_BLOCKS - 1);
  const int m = a.top_k - 1, n_c = local;
  int32_t *out = a.sel + pid * a.top_k;
  const unsigned char *rowb = reinterpret_cast<const unsigned char *>(a.bmax + pid * (long)a.n_blocks);
  const StridedIdx item{lane};
  auto block_of = [&](int32_t j) { return runs[j >> 5] * RUN_BLOCKS + (j & (RUN_BLOCKS - 1)); };
  uint32_t key[VI];
  float x[VI];
#pragma unroll
  for (int s = 0; s < VI; ++s) {
    const int blk = runs[min(2 * s + half, nr - 1)] * RUN_BLOCKS + sub;
    x[s] = __builtin_nontemporal_load(reinterpret_cast<const float *>(
        rowb + (uint32_t)min(blk, n_c - 1) * 4u));
  }
#pragma unroll
  for (int s = 0; s < VI; ++s) pin(x[s]);
#pragma unroll
  for (int s = 0; s < VI; ++s) {
    const int e = 2 * s + half;  // whole runs, then the tail's first tcount blocks
    key[s] = (e < cnt || (e < nr && sub < tcount)) ? order_key(x[s]) : 0u;
  }
  uint32_t ks = 0;
  int32_t is = 0x7fffffff;
  const int C = wave_threshold(key, item, m, lk, li, ks, is);  // at least 32 m items
  int pos = 0;
  if (C >= 0) {
    for (int q = 0; q * 64 < C; ++q) {
      const int j = q * 64 + lane;
      const uint32_t kv = j < C ? lk[j] : 0u;
      const int32_t iv = j < C ? li[j] : 0;
      const bool pr = taken(kv, iv, ks, is);
      const uint64_t mk = ballot(pr);
      if (pr) out[pos + rank_below(mk)] = block_of(iv);
      pos += popc64(mk);
    }
  } else {
#pragma unroll
    for (int s = 0; s < VI; ++s) {  // slot-major order is ascending block order
      const bool pr = taken(key[s], item[s], ks, is);
      const uint64_t mk = ballot(pr);
      if (pr) out[pos + rank_below(mk)] = block_of(item[s]);
      pos += popc64(mk);
    }
  }
  if (lane == 0) out[m] = local;
}

// One chunk of a problem (single: its only one, winners to sel; else to the candidates),
// with items per lane sized to the chunk's candidates (a wave-uniform choice).
__device__ __forceinline__ void select_sized(const TopkArgs &a, long pid, int chunk, int n_c,
                                             bool single, int local, uint32_t *lk, int32_t *li) {
  const int base = chunk * TOPK_CHUNK;
  const int valid = min(TOPK_CHUNK, n_c - base);
  if (valid <= 512)
    select_chunk<8>(a, pid, chunk, base, n_c, valid, single, local, lk, li);
  else if (valid <= 1024)
    select_chunk<16>(a, pid, chunk, base, n_c, valid, single, local, lk, li);
  else
    select_chunk<V>(a, pid, chunk, base, n_c, valid, single, local, lk, li);
}

// Every problem of a launch whose rows may exceed one chunk, with run keys. Grid: x = groups
// of 4 problems, one wave each; register budget as topk_pass1 for several chunks.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void topk_runs(TopkArgs a) {
  __shared__ uint32_t s_key[4][SELECT_LDS];
  __shared__ int32_t s_idx[4][SELECT_LDS];
  __shared__ int32_t s_run[4][64];
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const long n_prob = (long)a.batch * a.h_kv * a.n_q;
  const long pid = (long)blockIdx.x * 4 + w;
  if (pid >= n_prob) return;
  const int t = (int)(pid % a.n_q);
  const long p = (long)a.q_start + t;
  const int local = (int)(p / a.block_size);
  const int k = a.top_k, m = k - 1;
  int32_t *out = a.sel + pid * k;
  if (local + 1 <= k) {  // sees k blocks or fewer: all of them
    if (lane < k) out[lane] = lane <= local ? lane : -1;
    return;
  }
  if (m == 0) {  // top_k == 1: the local block alone
    if (lane == 0) out[0] = local;
    return;
  }
  const int n_c = local;  // candidates: blocks 0 .. local-1
  if (n_c <= TOPK_CHUNK) {
    select_sized(a, pid, 0, n_c, true, local, s_key[w], s_idx[w]);
    return;
  }
  const int nf = n_c / RUN_BLOCKS, tcount = n_c - nf * RUN_BLOCKS;  // nf > 64 > m
  const uint32_t *rrow = a.rkey + pid * (long)a.n_runs;
  int cnt = 65;  // more runs than phase 2 takes: the chunked path below
  if (nf <= 512)
    cnt = runs_at_bound<8>(rrow, nf, m, s_key[w], s_idx[w], s_run[w]);
  else if (nf <= 1024)
    cnt = runs_at_bound<16>(rrow, nf, m, s_key[w], s_idx[w], s_run[w]);
  else if (nf <= TOPK_CHUNK)
    cnt = runs_at_bound<V>(rrow, nf, m, s_key[w], s_idx[w], s_run[w]);
  const int nr = cnt + (tcount > 0 ? 1 : 0);
  // At least m runs reach the bound (always, unless a key is 0, the empty-slot mark, which
  // only a NaN input can give): else, as for too many runs, the chunked path.
  if (cnt >= m && nr <= 64) {
    if (tcount > 0 && lane == 0) s_run[w][cnt] = nf;  // the tail, after every whole run
    lds_wait();
    if (nr <= 16)
      rank_runs<8>(a, pid, local, s_run[w], cnt, nr, tcount, s_key[w], s_idx[w]);
    else if (nr <= 32)
      rank_runs<16>(a, pid, local, s_run[w], cnt, nr, tcount, s_key[w], s_idx[w]);
    else
      rank_runs<V>(a, pid, local, s_run[w], cnt, nr, tcount, s_key[w], s_idx[w]);
    return;
  }
  // Ties at the bound left too many runs (or the row has too many runs): the two passes,
  // in this wave. The merge reads back the candidates this wave's lanes wrote (through the
  // compute unit's own cache: a workgroup-scope fence orders them).
  const int nch = (n_c + TOPK_CHUNK - 1) / TOPK_CHUNK;
  for (int c = 0; c < nch; ++c) select_sized(a, pid, c, n_c, false, local, s_key[w], s_idx[w]);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the candidate stores have completed
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  merge_winners(a, pid, nch, local, s_key[w], s_idx[w], s_run[w]);
}

// Final merge for few problems with many candidates (decode: one problem per (sequence,
// group), the winners of every key range of the sequence): a workgroup of MW waves per
// problem runs the two stages of the wide merge and writes the winners in ascending block
// order, local block last.
constexpr int MW = 8;  // waves per problem

__global__ __launch_bounds__(MW * 64) void topk_merge_wide(TopkArgs a) {
  __shared__ uint32_t s_key[MW][SELECT_LDS];
  __shared__ int32_t s_idx[MW][SELECT_LDS];
  __shared__ uint32_t w_key[MW * 64];  // per-wave winners (MW * m used), padded with key 0
  __shared__ int32_t w_idx[MW * 64];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long pid = blockIdx.x;
  const int t = (int)(pid % a.n_q);
  const long p = (long)a.q_start + t;
  const int local = (int)(p / a.block_size);
  const int k = a.top_k, m = k - 1;
  int32_t *out = a.sel + pid * k;
  if (local + 1 <= k || m == 0) {  // sees k blocks or fewer, or k == 1 (uniform)
    if (w == 0) {
      if (local + 1 <= k) {
        if (lane < k) out[lane] = lane <= local ? lane : -1;
      } else if (lane == 0) {
        out[0] = local;
      }
    }
    return;
  }
  const int nch = (local + a.chunk_blocks - 1) / a.chunk_blocks;
  const int total = nch * m;  // <= TOPK_CHUNK (checked on the host)
  wide_stage1<MW>(a.cand_key + pid * a.n_chunks * (long)m, a.cand_idx + pid * a.n_chunks * (long)m,
                  total, m, w, s_key[w], s_idx[w], w_key, w_idx);
  __syncthreads();
  if (w != 0) return;
  wide_stage2<MW>(m, w_key, w_idx, s_key[0], s_idx[0], [&](int j, int32_t c) { out[j] = c; });
  if (lane == 0) out[m] = local;
}

}  // namespace

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
  const long n_prob = (long)a.batch * a.h_kv * a.n_q;
  const unsigned groups = (unsigned)((n_prob + 3) / 4);
  if (a.n_chunks > 1 && a.rkey) {
    hipLaunchKernelGGL(topk_runs, dim3(groups), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  if (a.n_chunks <= 1)
    hipLaunchKernelGGL(topk_pass1<6>, dim3(groups, 1u), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(topk_pass1<5>, dim3(groups, (unsigned)a.n_chunks), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_chunks <= 1) return e;
  hipLaunchKernelGGL(topk_pass2, dim3(groups), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topk_final(const TopkArgs &a, hipStream_t s) {
  const long n_prob = (long)a.batch * a.h_kv * a.n_q;
  hipLaunchKernelGGL(topk_merge_wide, dim3((unsigned)n_prob), dim3(MW * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace msa
