// msa_kvouter.hip -- main branch for prefill, organised KV-block-outer.
//
// The attention itself is the main-branch equation of "MiniMax-M3: MSA 技术报告速读"
// (section 核心机制): each head h of group r attends, for row t, to the visible tokens of
// the blocks in sel[b, r, t, :]. The organisation follows the kernel notes of the same
// page (section Kernel): every selected KV block gathers the query rows that chose it so
// the matrix cores see full tiles, and a fixed split with a second merge stage replaces
// atomic accumulation.
//
//   1. The list build inverts sel into per-(row segment, b, r, block) lists of
//      (row, slot) entries: per-workgroup LDS histograms, one workgroup's exclusive scan,
//      then a fill. Integer atomics only place entries; their order inside a list does not
//      change any result. Lists are keyed group-major, then by row segment, so that the
//      chunks processed at the same time share one group's K/V and a slice of its Q rows.
//   2. kv_attend (persistent, chunks claimed at run time): a workgroup takes chunks of up
//      to CHUNK entries of one list, stages the block's K (row-major) and V (transposed) in
//      LDS once, and each wave keeps
//      the block's K and V^T fragments in registers while it runs 16-row tiles (16/G rows
//      x the G heads of the group): S^T = K Q^T, a softmax over the block, O^T = V^T P^T.
//      It writes, for every (row, slot, head), the block's unnormalised output sum_j p_j v_j
//      and (m, l) with p_j = 2^(z_j - m), l = sum_j p_j (log2 units).
//   3. kv_merge: G * DH / 8 threads per (b, r, row) combine the row's partials in slot order
//      with weights 2^(m_s - M): O = sum_s w_s o_s / sum_s w_s l_s, LSE = (M + log2 L) ln 2.
#include "msa_device.hpp"
#include "msa_internal.hpp"

#include <algorithm>

namespace msa {
namespace {

constexpr int CHUNK = KV_CHUNK;           // entries per kv_attend work item
constexpr long KV_Q_SLICE = 64L << 20;    // bytes of one group's Q rows per list segment
constexpr int HIST_ROWS_ENTRIES = 32768;  // entries per list-build workgroup, at most
constexpr int HIST_MAX_BLOCKS = 32768;    // LDS histogram capacity (128 KiB)

// Rows per list-build workgroup: HIST_ROWS_ENTRIES entries, halved while the call would
// have fewer than 512 workgroups, so that short calls still spread the build over the chip
// (the 8K prefill had 16 workgroups), but not below 2048 entries nor below n_blocks: a
// histogram with fewer entries than bins holds mostly single counts, and its reservations
// become one global atomic per entry (the 1M-context chunk's build took 512 workgroups of
// 2048 entries over 16384 bins). Row segments are whole multiples of it, so a workgroup's
// rows lie in one segment.
__host__ __device__ __forceinline__ long hist_tile_rows(long batch, long h_kv, long n_q, long top_k,
                                                        long n_blocks) {
  const long total = batch * h_kv * n_q * top_k;
  const long least = n_blocks > 2048 ? n_blocks : 2048;
  long ent = HIST_ROWS_ENTRIES;
  while (ent > least && total / ent < 512) ent >>= 1;
  return ent / top_k > 1 ? ent / top_k : 1;
}

__global__ void fill_i32(int32_t *p, long n, int32_t v) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    p[i] = v;
}

// List index of (b, r, row t, block c): group-major, then row segment, then sequence. The
// chunks in flight at one time then share one group's K/V and one segment's Q rows of that
// group, which fit together in the 256 MB memory-side cache (64 MiB of each at 128K rows).
// Smaller segments would keep Q in L2 but cut the rows per list, and so the reuse of each
// staged K/V block: measured slower.
__device__ __forceinline__ long list_index(const KvArgs &a, long br, int t, int c) {
  const long seg = t / a.seg_rows;
  const long r = br % a.h_kv, b = br / a.h_kv;
  return ((r * a.n_seg + seg) * a.batch + b) * a.n_blocks + c;
}

// ---------------------------------------------------------------- list build

// Fallback for more blocks than an LDS histogram holds: one counter update per entry.
__global__ __launch_bounds__(256) void kv_count(KvArgs a) {
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  const long total = (long)a.batch * a.h_kv * a.n_q * a.top_k;
  if (e >= total) return;
  const int c = a.sel[e];
  if (c < 0 || c >= a.n_blocks) return;
  const long row = e / a.top_k;
  atomicAdd(&a.cnt[list_index(a, row / a.n_q, (int)(row % a.n_q), c)], 1);
}

__global__ __launch_bounds__(256) void kv_fill(KvArgs a) {
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  const long total = (long)a.batch * a.h_kv * a.n_q * a.top_k;
  if (e >= total) return;
  const int c = a.sel[e];
  if (c < 0 || c >= a.n_blocks) return;
  const long row = e / a.top_k;
  const int t = (int)(row % a.n_q);
  const long i = list_index(a, row / a.n_q, t, c);
  const int pos = a.boff[i] + atomicAdd(&a.cursor[i], 1);
  a.list[pos] = t * 64 + (int)(e % a.top_k);
}


// Rows of this list-build workgroup (they lie in one row segment); `base` is the list
// index of block 0 for them.
__device__ __forceinline__ void hist_rows(const KvArgs &a, long &e_begin, long &e_end, long &base) {
  const long rows_per_wg = hist_tile_rows(a.batch, a.h_kv, a.n_q, a.top_k, a.n_blocks);
  const long tiles_per_br = (a.n_q + rows_per_wg - 1) / rows_per_wg;
  const long br = blockIdx.x / tiles_per_br;
  const long r0 = (blockIdx.x % tiles_per_br) * rows_per_wg;
  const long r1 = min((long)a.n_q, r0 + rows_per_wg);
  e_begin = (br * a.n_q + r0) * a.top_k;
  e_end = (br * a.n_q + r1) * a.top_k;
  base = list_index(a, br, (int)r0, 0);
}

__global__ __launch_bounds__(1024) void kv_count_hist(KvArgs a) {
  extern __shared__ int32_t s_hist[];
  long e0, e1, base;
  hist_rows(a, e0, e1, base);
  for (int c = threadIdx.x; c < a.n_blocks; c += 1024) s_hist[c] = 0;
  __syncthreads();
  for (long e = e0 + threadIdx.x; e < e1; e += 1024) {
    const int c = a.sel[e];
    if (c >= 0 && c < a.n_blocks) atomicAdd(&s_hist[c], 1);
  }
  __syncthreads();
  for (int c = threadIdx.x; c < a.n_blocks; c += 1024)
    if (s_hist[c]) atomicAdd(&a.cnt[base + c], s_hist[c]);
}

__global__ __launch_bounds__(1024) void kv_fill_hist(KvArgs a) {
  extern __shared__ int32_t s_hist[];
  long e0, e1, base;
  hist_rows(a, e0, e1, base);
  for (int c = threadIdx.x; c < a.n_blocks; c += 1024) s_hist[c] = 0;
  __syncthreads();
  for (long e = e0 + threadIdx.x; e < e1; e += 1024) {
    const int c = a.sel[e];
    if (c >= 0 && c < a.n_blocks) atomicAdd(&s_hist[c], 1);
  }
  __syncthreads();
  for (int c = threadIdx.x; c < a.n_blocks; c += 1024) {  // reserve this workgroup's ranges
    const int n = s_hist[c];
    if (n) s_hist[c] = a.boff[base + c] + atomicAdd(&a.cursor[base + c], n);
  }
  __syncthreads();
  for (long e = e0 + threadIdx.x; e < e1; e += 1024) {
    const int c = a.sel[e];
    if (c >= 0 && c < a.n_blocks) {
      const int pos = atomicAdd(&s_hist[c], 1);
      a.list[pos] = (int)((e / a.top_k) % a.n_q) * 64 + (int)(e % a.top_k);
    }
  }
}

// Exclusive scans of the per-list entry counts and chunk counts, and the chunk -> list map,
// in three parallel phases over tiles of SCAN_TILE lists: tile sums, one scan of the tile
// sums, then each tile's own scan with its offset.
constexpr int SCAN_TILE = 1024;  // lists per scan workgroup (256 threads x 4)

__device__ __forceinline__ int chunks_of(int n) { return (n + CHUNK - 1) / CHUNK; }

// Block-wide exclusive scan of one value per thread (256 threads); returns the total.
__device__ __forceinline__ long block_excl_scan(long v, long &excl, long *s_w) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  long incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) s_w[w] = incl;
  __syncthreads();
  long base = 0, total = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < w) base += s_w[i];
    total += s_w[i];
  }
  __syncthreads();
  excl = base + incl - v;
  return total;
}

__global__ __launch_bounds__(256) void kv_scan_tiles(KvArgs a) {
  __shared__ long s_w[2][4];
  const long NB = (long)a.n_seg * a.batch * a.h_kv * a.n_blocks;
  const long i0 = (long)blockIdx.x * SCAN_TILE + threadIdx.x * 4;
  long sp = 0, sc = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (i0 + u < NB) {
      const int n = a.cnt[i0 + u];
      sp += n;
      sc += chunks_of(n);
    }
  long ep, ec;
  const long tp = block_excl_scan(sp, ep, s_w[0]);
  const long tc = block_excl_scan(sc, ec, s_w[1]);
  if (threadIdx.x == 0) {
    a.tile_sum[2 * blockIdx.x] = tp;
    a.tile_sum[2 * blockIdx.x + 1] = tc;
  }
}

// One workgroup: exclusive scan of the tile sums in place; writes the totals.
__global__ __launch_bounds__(256) void kv_scan_top(KvArgs a) {
  __shared__ long s_w[2][4];
  const long NB = (long)a.n_seg * a.batch * a.h_kv * a.n_blocks;
  const long n_tiles = (NB + SCAN_TILE - 1) / SCAN_TILE;
  long carry_p = 0, carry_c = 0;
  for (long base = 0; base < n_tiles; base += 256) {
    const long i = base + threadIdx.x;
    const long vp = i < n_tiles ? a.tile_sum[2 * i] : 0, vc = i < n_tiles ? a.tile_sum[2 * i + 1] : 0;
    long ep, ec;
    const long tp = block_excl_scan(vp, ep, s_w[0]);
    const long tc = block_excl_scan(vc, ec, s_w[1]);
    if (i < n_tiles) {
      a.tile_sum[2 * i] = carry_p + ep;
      a.tile_sum[2 * i + 1] = carry_c + ec;
    }
    carry_p += tp;
    carry_c += tc;
  }
  if (threadIdx.x == 0) {
    a.boff[NB] = (int32_t)carry_p;
    a.coff[NB] = (int32_t)carry_c;
  }
}

__global__ __launch_bounds__(256) void kv_scan_apply(KvArgs a) {
  __shared__ long s_w[2][4];
  const long NB = (long)a.n_seg * a.batch * a.h_kv * a.n_blocks;
  const long i0 = (long)blockIdx.x * SCAN_TILE + threadIdx.x * 4;
  int n[4];
  long sp = 0, sc = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    n[u] = i0 + u < NB ? a.cnt[i0 + u] : 0;
    sp += n[u];
    sc += chunks_of(n[u]);
  }
  long ep, ec;
  block_excl_scan(sp, ep, s_w[0]);
  block_excl_scan(sc, ec, s_w[1]);
  long rp = a.tile_sum[2 * blockIdx.x] + ep, rc = a.tile_sum[2 * blockIdx.x + 1] + ec;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (i0 + u < NB) {
      a.boff[i0 + u] = (int32_t)rp;
      a.coff[i0 + u] = (int32_t)rc;
      for (int j = 0; j < chunks_of(n[u]); ++j) a.cmap[rc + j] = (int32_t)(i0 + u);
      rp += n[u];
      rc += chunks_of(n[u]);
    }
}

// ---------------------------------------------------------------- attention per block

// LDS layout of a staged block. The matrix-core fragment reads of K take 16-byte pieces:
// in each pass of the LDS, 16 lanes read rows 0-7 at piece p and rows 8-15 at piece p + 1,
// and those 16 pieces must fall on distinct 16-byte bank groups (the 64 banks hold 16).
//   bf16, 256-byte K rows of 64-key blocks: unpadded, the piece XORed by 2 * (row & 7):
//     rows 0-7 take the 8 pieces of p's parity, rows 8-15 the other 8, with no LDS spent
//     on padding (that kernel holds three workgroups per compute unit only within this
//     budget). The XOR costs a VGPR per piece address, so it is used only there.
//   bf16, other K rows: padded by 32 bytes, which places rows 0-7 and 8-15 on the even
//     and odd bank groups.
//   bf16 V^T rows padded by 8 bytes: the two 8-byte halves of a fragment, 32 bytes apart,
//     are read by one ds_read2_b64, which measured free of bank conflicts at this pitch
//     (and at 7.5 conflict cycles per instruction with 16 bytes of padding).
template <typename E, int DH, int BS>
struct KvLds {
  static constexpr int ES = (int)sizeof(E);
  static constexpr bool KSWZ = ES == 2 && DH * ES == 256 && BS == 64;
  static constexpr int KROW = KSWZ ? DH * ES : DH * ES + (ES == 2 ? 32 : 16);  // K row-major
  static constexpr int VROW = BS * ES + (ES == 2 ? 8 : 16);  // V^T rows (one per d)
  static constexpr int K_BYTES = BS * KROW;
  static constexpr int V_BYTES = DH * VROW;
  // byte offset of 16-byte piece `piece` of K row `row`
  __device__ static __forceinline__ int k_at(int row, int piece) {
    return row * KROW + (KSWZ ? piece ^ (2 * (row & 7)) : piece) * 16;
  }
};

// Stage block rows [kb, kb+BS) of K (row-major) and V (transposed) into LDS, 256 threads.
// Every load of the block is issued before the first LDS write: rows past n_k read row
// n_k - 1 instead (their keys are masked and their probabilities are 0), so no load sits
// under a branch, which would make each wait for the one before. bf16 loads are
// non-temporal: a block is staged once per chunk and its lines are not worth keeping in L2
// over the Q rows the chunks gather.
template <typename E, int DH, int BS>
__device__ __forceinline__ void stage_block(const E *kp, const E *vp, long kb, int n_k,
                                            unsigned char *ks, unsigned char *vt) {
  using L = KvLds<E, DH, BS>;
  const int tid = threadIdx.x;
  constexpr int KPIECES = BS * DH * L::ES / 16;
  constexpr int PER_ROW = DH * L::ES / 16;
  constexpr int KPT = (KPIECES + 255) / 256;
  const long last = (long)n_k - 1;
  u32x4 kx[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int pc = min(tid + 256 * i, KPIECES - 1);
    const long j = min(kb + pc / PER_ROW, last);
    kx[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
        reinterpret_cast<const unsigned char *>(kp + j * DH) + (pc % PER_ROW) * 16));
  }
  if constexpr (L::ES == 2) {
    constexpr int PAIRS = BS / 2, VPIECES = PAIRS * (DH / 8);
    constexpr int VPT = (VPIECES + 255) / 256;
    u32x4 vx[VPT], vy[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int pc = min(tid + 256 * i, VPIECES - 1);
      const int kpair = pc % PAIRS, d0 = (pc / PAIRS) * 8;
      const long j0 = min(kb + 2 * kpair, last), j1 = min(kb + 2 * kpair + 1, last);
      vx[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vp + j0 * DH + d0));
      vy[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vp + j1 * DH + d0));
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) pin(kx[i]);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      pin(vx[i]);
      pin(vy[i]);
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int pc = tid + 256 * i;
      if (KPIECES % 256 == 0 || pc < KPIECES)
        *reinterpret_cast<u32x4 *>(ks + L::k_at(pc / PER_ROW, pc % PER_ROW)) = kx[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int pc = tid + 256 * i;
      if (VPIECES % 256 == 0 || pc < VPIECES) {
        const int kpair = pc % PAIRS, d0 = (pc / PAIRS) * 8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t x = vx[i][e], y = vy[i][e];
          *reinterpret_cast<uint32_t *>(vt + (d0 + 2 * e) * L::VROW + kpair * 4) = (x & 0xffffu) | (y << 16);
          *reinterpret_cast<uint32_t *>(vt + (d0 + 2 * e + 1) * L::VROW + kpair * 4) = (x >> 16) | (y & 0xffff0000u);
        }
      }
    }
  } else {
    constexpr int VPIECES = BS * (DH / 4);
    constexpr int VPT = (VPIECES + 255) / 256;
    f32x4 vx[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int pc = min(tid + 256 * i, VPIECES - 1);
      const long j = min(kb + pc % BS, last);
      vx[i] = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(vp) + j * DH + (pc / BS) * 4);
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) pin(kx[i]);
#pragma unroll
    for (int i = 0; i < VPT; ++i) pin(vx[i]);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int pc = tid + 256 * i;
      if (KPIECES % 256 == 0 || pc < KPIECES)
        *reinterpret_cast<u32x4 *>(ks + L::k_at(pc / PER_ROW, pc % PER_ROW)) = kx[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int pc = tid + 256 * i;
      if (VPIECES % 256 == 0 || pc < VPIECES) {
        const int key = pc % BS, d0 = (pc / BS) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) *reinterpret_cast<float *>(vt + (d0 + e) * L::VROW + key * 4) = vx[i][e];
      }
    }
  }
}

// V^T fragment for d-row `row` and 32-key step ks: keys 32ks+4g+0..3, then 32ks+16+4g+0..3
// (the order in which the S^T accumulators hold P^T).
__device__ __forceinline__ bf16x8 vt_frag(const unsigned char *row, int ks, int g, const bf16_t *) {
  const u32x2 lo = *reinterpret_cast<const u32x2 *>(row + (32 * ks + 4 * g) * 2);
  const u32x2 hi = *reinterpret_cast<const u32x2 *>(row + (32 * ks + 16 + 4 * g) * 2);
  return __builtin_bit_cast(bf16x8, (u32x4{lo[0], lo[1], hi[0], hi[1]}));
}
__device__ __forceinline__ f32x8 vt_frag(const unsigned char *row, int ks, int g, const float *) {
  const f32x4 lo = *reinterpret_cast<const f32x4 *>(row + (32 * ks + 4 * g) * 4);
  const f32x4 hi = *reinterpret_cast<const f32x4 *>(row + (32 * ks + 16 + 4 * g) * 4);
  return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ bf16x8 pt_frag(f32x4 a, f32x4 b, const bf16_t *) {
  return __builtin_bit_cast(bf16x8, (u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                           pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])}));
}
__device__ __forceinline__ f32x8 pt_frag(f32x4 a, f32x4 b, const float *) {
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ void store4(bf16_t *dst, f32x4 v) {
  *reinterpret_cast<u32x2 *>(dst) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
__device__ __forceinline__ void store4(float *dst, f32x4 v) { *reinterpret_cast<f32x4 *>(dst) = v; }

// Each wave reads the block's K and V^T fragments from LDS per tile (keeping them in
// registers across tiles cost resident waves and was not kept).
template <typename E, int DH, int BS>
__global__ __launch_bounds__(256) void kv_attend(KvArgs a, int log2g) {
  using F = typename Frag<E>::type;
  using L = KvLds<E, DH, BS>;
  constexpr int DC = DH / 32, KTN = BS / 16, DT = DH / 16, KS = BS / 32;
  constexpr int OROW = DH * L::ES + 16;  // one output row in the store-staging buffer
  __shared__ __attribute__((aligned(16))) unsigned char s_k[L::K_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char s_v[L::V_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char s_o[4][16 * OROW];  // per wave
  __shared__ int32_t s_list[CHUNK];
  // A chunk's list is loaded by a loop over its entries (any CHUNK), but the tiles below
  // assume the 256-thread workgroup that every CHUNK up to 256 has been tested with.
  static_assert(CHUNK <= 256, "kv_attend: chunks longer than the workgroup are untested");

  const long NB = (long)a.n_seg * a.batch * a.h_kv * a.n_blocks;
  const int n_chunks = a.coff[NB];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int G = 1 << log2g, QPT = 16 >> log2g;
  const int qi = c16 >> log2g, hd = c16 & (G - 1);
  const E *q = reinterpret_cast<const E *>(a.q);
  const float cs = a.scale_log2;

  __shared__ int s_next;
  for (int chunk = blockIdx.x; chunk < n_chunks; chunk = s_next) {  // uniform loop
    const long i = a.cmap[chunk];
    const int c = (int)(i % a.n_blocks);
    const long rsb = i / a.n_blocks;  // (r, seg, b) of the list
    const int b = (int)(rsb % a.batch);
    const int r = (int)(rsb / a.batch / a.n_seg);
    const int e0 = a.boff[i] + (chunk - a.coff[i]) * CHUNK;
    const int n_e = min(e0 + CHUNK, a.boff[i + 1]) - e0;
    const long plane = ((long)b * a.h_kv + r) * (long)a.cap * DH;
    const E *kp = reinterpret_cast<const E *>(a.k) + plane;
    const E *vp = reinterpret_cast<const E *>(a.v) + plane;
    const long kb = (long)c * BS;
    const int h = r * G + hd;

    __syncthreads();  // the previous chunk is done with the LDS buffers and s_next
    if (tid == 0) s_next = claim_next(a.claim, n_chunks);
    for (int e = tid; e < n_e; e += 256) s_list[e] = a.list[e0 + e];  // any CHUNK
    stage_block<E, DH, BS>(kp, vp, kb, a.n_k, s_k, s_v);
    __syncthreads();


    const int n_tiles = (n_e + QPT - 1) / QPT;
    // Q rows of tile tt. The loads are unconditional (lanes past the chunk's entries read
    // the first entry's row; their columns are masked and never stored) so that the
    // prefetch of the next tile stays in flight: a load under a branch makes the compiler
    // wait for every outstanding load before the next use of any of them.
    auto load_q = [&](int tt, F (&dst)[DC]) {
      const int e = tt * QPT + qi;
      const int t = s_list[(tt < n_tiles && e < n_e) ? e : 0] >> 6;
      const E *src = q + (((long)b * a.h_q + h) * a.n_q + t) * DH + g * 8;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) dst[dc] = load_frag(src + dc * 32);
    };
    F bq[DC], bq_next[DC];
    load_q(w, bq);
    for (int tt = w; tt < n_tiles; tt += 4) {
      load_q(tt + 4, bq_next);  // in flight while this tile computes
      const int e = tt * QPT + qi;
      const bool valid = e < n_e;
      const int ent = valid ? s_list[e] : 0;
      const int t = ent >> 6, slot = ent & 63;
      const long p = (long)a.q_start + t;

      f32x4 s[KTN];
#pragma unroll
      for (int kt = 0; kt < KTN; ++kt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          const F af = load_frag(reinterpret_cast<const E *>(
              s_k + L::k_at(kt * 16 + c16, (dc * 32 + g * 8) * L::ES / 16)));
          acc = mfma_chunk(af, bq[dc], acc);
        }
        s[kt] = acc;
      }
      // Rows that need masking (their own block, or no entry) are rare: one uniform test.
      const bool fix = !valid || kb + BS - 1 > p;
      if (ballot(fix)) {
        const int lim = valid ? (int)min(p - kb, (long)BS) : -1;  // key offset visible iff <= lim
#pragma unroll
        for (int kt = 0; kt < KTN; ++kt)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
            if (kt * 16 + g * 4 + ii > lim) s[kt][ii] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < KTN; ++kt) mx = fmaxf(mx, fmaxf(fmaxf(s[kt][0], s[kt][1]), fmaxf(s[kt][2], s[kt][3])));
      mx = max_groups(mx);
      const float m = mx == -INFINITY ? 0.f : mx * cs;  // log2 units
      float rs = 0.f;
#pragma unroll
      for (int kt = 0; kt < KTN; ++kt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float pz = __builtin_amdgcn_exp2f(fmaf(s[kt][ii], cs, -m));  // exp2(-inf) = 0
          s[kt][ii] = pz;
          rs += pz;
        }
      rs = sum_groups(rs);
      f32x4 o[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const F bp = pt_frag(s[2 * ks], s[2 * ks + 1], kp);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const F av = vt_frag(s_v + (dt * 16 + c16) * L::VROW, ks, g, kp);
          o[dt] = mfma_chunk(av, bp, o[dt]);
        }
      }
      // Stage the tile's 16 output rows in LDS, then write each entry's G x DH block with
      // contiguous 16-byte pieces (consecutive lanes, consecutive addresses), non-temporal:
      // the merge reads them once, long after.
      unsigned char *so = s_o[w];
      if constexpr (L::ES == 2) {
        // Lane (c16, g) holds d = 16 dt + 4 g + 0..3 of row-head c16. Lane groups g and g ^ 1
        // swap halves (v_permlane16_swap pairs the odd 16-lane rows of its first operand
        // with the even rows of its second), after which even groups hold the 8 consecutive
        // d from 16 dt + 4 g of tile dt and odd groups those from 16 (dt + 1) + 4 (g - 1) of
        // tile dt + 1: one 16-byte store each. Pairs of 8-byte stores merge into
        // ds_write2_b64, which measured 7.5 bank-conflict cycles per instruction here.
        static_assert(DT % 2 == 0, "output tiles are stored in pairs");
#pragma unroll
        for (int dt = 0; dt < DT; dt += 2) {
          const auto lo = __builtin_amdgcn_permlane16_swap(pack_bf16x2(o[dt][0], o[dt][1]),
                                                           pack_bf16x2(o[dt + 1][0], o[dt + 1][1]), false, false);
          const auto hi = __builtin_amdgcn_permlane16_swap(pack_bf16x2(o[dt][2], o[dt][3]),
                                                           pack_bf16x2(o[dt + 1][2], o[dt + 1][3]), false, false);
          const int d0 = (g & 1) ? 16 * (dt + 1) + 4 * (g - 1) : 16 * dt + 4 * g;
          *reinterpret_cast<u32x4 *>(so + c16 * OROW + d0 * 2) = u32x4{lo[0], hi[0], lo[1], hi[1]};
        }
      } else {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) store4(reinterpret_cast<E *>(so + c16 * OROW) + dt * 16 + g * 4, o[dt]);
      }
      if (valid && g == 0) {
        const long ps = ((((long)b * a.h_kv + r) * a.n_q + t) * a.top_k + slot) * G + hd;
        reinterpret_cast<float2 *>(a.part_ml)[ps] = make_float2(rs > 0.f ? m : -INFINITY, rs);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // wave-private buffer: in-order LDS
      {
        // A fixed number of stores per lane with no branch, so that the compiler counts
        // them and the next tile's wait for its Q fragments (loaded before these stores)
        // leaves them in flight. Rows past the chunk's entries store the tile's first row
        // of the same head again (the same bytes to the same address).
        constexpr int PIECES_ROW = DH * L::ES / 16;  // 16-byte pieces per output row
        constexpr int NST = 16 * PIECES_ROW / 64;    // the whole tile, per lane
        static_assert(16 * PIECES_ROW % 64 == 0, "output pieces must fill whole waves");
        // With 17-piece rows (256-byte rows padded by 16), piece p of row rw sits on bank
        // group (rw + p) % 16. Lanes of row lane / 16 + 4 i take piece lane - lane / 16,
        // which lies on bank group lane + 4 i, so the 16 lanes of an LDS pass (two rows)
        // cover all 16 groups, with one address per lane for every i.
        constexpr bool ROT = PIECES_ROW == 16 && OROW == 17 * 16;
        u32x4 val[NST];
        u32x4 *dst[NST];
#pragma unroll
        for (int i = 0; i < NST; ++i) {
          const int pc = lane + 64 * i;
          int row = pc / PIECES_ROW;
          const int off = ROT ? (lane - (lane >> 4)) & 15 : pc % PIECES_ROW;
          if (tt * QPT + (row >> log2g) >= n_e) row &= G - 1;
          const int en = s_list[tt * QPT + (row >> log2g)];
          const long pss = ((((long)b * a.h_kv + r) * a.n_q + (en >> 6)) * a.top_k + (en & 63)) * G + (row & (G - 1));
          val[i] = *reinterpret_cast<const u32x4 *>(so + row * OROW + off * 16);
          dst[i] = reinterpret_cast<u32x4 *>(reinterpret_cast<unsigned char *>(a.part_o) + pss * DH * L::ES + off * 16);
        }
#pragma unroll
        for (int i = 0; i < NST; ++i) __builtin_nontemporal_store(val[i], dst[i]);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) bq[dc] = bq_next[dc];
    }
  }
}

// ---------------------------------------------------------------- merge

// 8 partial-output elements of one (slot, head), packed as stored (read once: non-temporal).
template <typename E> struct Raw8;
template <> struct Raw8<bf16_t> {
  u32x4 x;
  __device__ __forceinline__ void load(const bf16_t *p) { x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p)); }
  __device__ __forceinline__ float operator[](int e) const {
    const uint32_t u = x[e >> 1];
    return __uint_as_float((e & 1) ? (u & 0xffff0000u) : (u << 16));
  }
};
template <> struct Raw8<float> {
  f32x4 lo, hi;
  __device__ __forceinline__ void load(const float *p) {
    lo = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    hi = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p + 4));
  }
  __device__ __forceinline__ float operator[](int e) const { return e < 4 ? lo[e] : hi[e - 4]; }
};

// Each (b, r, row) is merged by LPR = G * DH / 8 consecutive threads (a wave holds several
// rows when LPR < 64; a row spans LPR / 64 waves otherwise); a thread owns 8 consecutive
// outputs of one head. Slots are taken U at a time with their loads in flight together.
template <typename E, int DH, int U>
__global__ __launch_bounds__(256) void kv_merge(KvArgs a, int log2g) {
  const int G = 1 << log2g;
  const int lpr_log2 = log2g + (DH == 128 ? 4 : 3);
  const int span = min(1 << lpr_log2, 64);  // lanes of one row inside a wave
  const long gl = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = gl >> lpr_log2;          // (b, r, t)
  const long rows = (long)a.batch * a.h_kv * a.n_q;
  const int lane = threadIdx.x & 63;
  const int j = (int)(gl & ((1L << lpr_log2) - 1));

  // valid slots of this row (top_k <= 64): ballots over the row's lanes, span slots a round
  uint64_t mask = 0;
  for (int m = 0; m * span < a.top_k; ++m) {
    const int sl = m * span + (lane & (span - 1));
    const int c = (sl < a.top_k && row < rows) ? a.sel[row * a.top_k + sl] : -1;
    const uint64_t bl = ballot(c >= 0 && c < a.n_blocks);
    const uint64_t bits = span == 64 ? bl : ((bl >> (lane & ~(span - 1))) & ((1ull << span) - 1));
    mask |= bits << (m * span);
  }
  if (row >= rows) return;  // no cross-lane work below

  const int hd = j / (DH / 8), d0 = (j % (DH / 8)) * 8;
  const float2 *ml = reinterpret_cast<const float2 *>(a.part_ml) + row * a.top_k * G + hd;
  const E *pbase = reinterpret_cast<const E *>(a.part_o) + (row * a.top_k * G + hd) * DH + d0;
  float acc[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) acc[x] = 0.f;
  float M = -INFINITY, Ls = 0.f;
  uint64_t v = mask;
  while (v) {
    int sl[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      sl[u] = v ? __builtin_ctzll(v) : -1;
      v &= v - 1;  // no-op once v is 0
    }
    float2 mls[U];
    Raw8<E> part[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      mls[u] = sl[u] >= 0 ? ml[(long)sl[u] * G] : make_float2(-INFINITY, 0.f);
      if (sl[u] >= 0) part[u].load(pbase + (long)sl[u] * G * DH);
    }
    float Mb = M;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (mls[u].y > 0.f) Mb = fmaxf(Mb, mls[u].x);
    const float sc = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mb);  // rescale earlier slots
    Ls *= sc;
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[x] *= sc;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (mls[u].y > 0.f) {
        const float wgt = __builtin_amdgcn_exp2f(mls[u].x - Mb);
        Ls += wgt * mls[u].y;
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[x] += wgt * part[u][x];
      }
    }
    M = Mb;
  }
  const int t = (int)(row % a.n_q);
  const long br = row / a.n_q;
  const int r = (int)(br % a.h_kv), b = (int)(br / a.h_kv);
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
  E *o = reinterpret_cast<E *>(a.o) + (((long)b * a.h_q + r * G + hd) * a.n_q + t) * DH + d0;
  store4(o, f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv});
  store4(o + 4, f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv});
  if (a.lse && d0 == 0)
    a.lse[((long)b * a.h_q + r * G + hd) * a.n_q + t] = (M + __log2f(Ls)) * 0.69314718055994531f;
}

void scan(const KvArgs &a, long NB, hipStream_t s) {
  const unsigned tiles = (unsigned)((NB + SCAN_TILE - 1) / SCAN_TILE);
  hipLaunchKernelGGL(kv_scan_tiles, dim3(tiles), dim3(256), 0, s, a);
  hipLaunchKernelGGL(kv_scan_top, dim3(1), dim3(256), 0, s, a);
  hipLaunchKernelGGL(kv_scan_apply, dim3(tiles), dim3(256), 0, s, a);
}

template <typename E, int DH, int BS>
hipError_t run_kv(const KvArgs &a, int log2g, int stages, hipStream_t s) {
  const long NB = (long)a.n_seg * a.batch * a.h_kv * a.n_blocks;
  const long entries = (long)a.batch * a.h_kv * a.n_q * a.top_k;
  if (stages & KV_STAGE_PLAN) {
    hipLaunchKernelGGL(fill_i32, dim3((unsigned)std::min(4096L, (2 * NB + 1 + 255) / 256)), dim3(256), 0, s,
                       a.cnt, 2 * NB + 1, 0);  // cnt, cursor and the claim counter are adjacent
    // per-workgroup LDS histograms while the device's LDS per workgroup holds n_blocks
    // counters; per-entry global counters otherwise
    static const long lds_max = [] {
      int dev = 0, v = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
        v = 64 << 10;
      return (long)v;
    }();
    if (a.n_blocks <= HIST_MAX_BLOCKS && (long)a.n_blocks * (long)sizeof(int32_t) <= lds_max) {
      const long rows_per_wg = hist_tile_rows(a.batch, a.h_kv, a.n_q, a.top_k, a.n_blocks);  // divides seg_rows
      const unsigned wgs = (unsigned)((long)a.batch * a.h_kv * ((a.n_q + rows_per_wg - 1) / rows_per_wg));
      const size_t lds = (size_t)a.n_blocks * sizeof(int32_t);
      hipLaunchKernelGGL(kv_count_hist, dim3(wgs), dim3(1024), lds, s, a);
      scan(a, NB, s);
      hipLaunchKernelGGL(kv_fill_hist, dim3(wgs), dim3(1024), lds, s, a);
    } else {
      const unsigned eg = (unsigned)((entries + 255) / 256);
      hipLaunchKernelGGL(kv_count, dim3(eg), dim3(256), 0, s, a);
      scan(a, NB, s);
      hipLaunchKernelGGL(kv_fill, dim3(eg), dim3(256), 0, s, a);
    }
  }
  if (stages & KV_STAGE_ATTEND) {
    // persistent: a few workgroups per CU loop over the chunks
    static const int per_cu = [] {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kv_attend<E, DH, BS>, 256, 0) !=
              hipSuccess || n < 1)
        n = 1;
      return n;
    }();
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    // one round of the workgroups that fit on the device at once; chunks are claimed
    const long max_chunks = (entries + CHUNK - 1) / CHUNK + NB;
    const unsigned grid = (unsigned)std::min(max_chunks, (long)per_cu * cus);
    KvArgs b = a;
    b.claim = a.cnt + 2 * NB;
    hipLaunchKernelGGL((kv_attend<E, DH, BS>), dim3(grid), dim3(256), 0, s, b, log2g);
  }
  if (!(stages & KV_STAGE_MERGE)) return hipGetLastError();
  const long threads = (long)a.batch * a.h_kv * a.n_q * ((long)DH << log2g) / 8;
  hipLaunchKernelGGL((kv_merge<E, DH, 32>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     a, log2g);
  return hipGetLastError();
}

}  // namespace

int kv_segment_rows(long batch, long h_kv, long n_q, long top_k, long n_blocks, long group,
                    long d_h, long elem_bytes) {
  // about KV_Q_SLICE bytes of one group's Q rows per segment, in whole list-build tiles
  const long tile = hist_tile_rows(batch, h_kv, n_q, top_k, n_blocks);
  const long per_row = group * d_h * elem_bytes;
  long rows = std::max(1L, KV_Q_SLICE / per_row);
  rows = std::max(tile, rows / tile * tile);
  return (int)std::min(rows, ((n_q + tile - 1) / tile) * tile);
}

size_t kv_workspace_bytes(long batch, long h_kv, long n_q, long top_k, long n_blocks, long group,
                          long d_h, long elem_bytes, KvLayout *lay) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const long seg_rows = kv_segment_rows(batch, h_kv, n_q, top_k, n_blocks, group, d_h, elem_bytes);
  const long n_seg = (n_q + seg_rows - 1) / seg_rows;
  const size_t NB = (size_t)(n_seg * batch * h_kv * n_blocks);
  const size_t slots = (size_t)(batch * h_kv * n_q * top_k);
  const size_t max_chunks = (slots + CHUNK - 1) / CHUNK + NB;
  KvLayout L;
  size_t o = 0;
  L.cnt = o;     o += al((2 * NB + 1) * 4);  // cnt, then cursor, then the chunk claim counter
  L.boff = o;    o += al((NB + 1) * 4);
  L.coff = o;    o += al((NB + 1) * 4);
  L.cmap = o;    o += al(max_chunks * 4);
  L.tile_sum = o; o += al(2 * ((NB + SCAN_TILE - 1) / SCAN_TILE) * 8);
  L.list = o;    o += al(slots * 4);
  L.part_o = o;  o += al(slots * (size_t)group * (size_t)d_h * (size_t)elem_bytes);
  L.part_ml = o; o += al(slots * (size_t)group * 8);
  L.total = o;
  if (lay) *lay = L;
  return o;
}

hipError_t launch_attn_prefill_kv(const KvArgs &a, int dtype, int d_h, int stages, hipStream_t s) {
  int lg = 0;
  while ((1 << lg) < a.h_q / a.h_kv) ++lg;
#define MSA_KV(E, DH)                                                             \
  if (a.block_size == 32) return run_kv<E, DH, 32>(a, lg, stages, s);                     \
  return run_kv<E, DH, 64>(a, lg, stages, s);
  if (dtype == 0) {
    if (d_h == 64) { MSA_KV(float, 64) }
    MSA_KV(float, 128)
  }
  if (d_h == 64) { MSA_KV(bf16_t, 64) }
  MSA_KV(bf16_t, 128)
#undef MSA_KV
}

}  // namespace msa
