// msa_kl.hip -- the index branch's alignment loss over the selected tokens.
//
// Definition ("MiniMax-M3: MSA 技术报告速读", section 训练, the equations for P^idx, P^(r)
// and L_KL): for row t of group r, over the selected blocks' visible tokens T,
//   student  P^idx_j = softmax_T(S^idx)_j,  S^idx_j = q_idx . k_idx_j / sqrt(d_idx)
//   teacher  P^(r)_j = (1/G) sum over the group's heads l of softmax_T(S^(l))_j,
//            S^(l)_j = q_l . k_j / sqrt(d_h)
//   L_KL = KL(P^(r) || P^idx) = sum_j P^(r)_j (ln P^(r)_j - ln P^idx_j).
// The teacher uses the main branch's log-sum-exp from the forward pass (the same page's
// Kernel section has the sparse loss take it from the forward), so each head's
// probabilities are exp(S^(l)_j - lse_l) with no second normalisation pass.
//
// Organised like the prefill attention, KV-block-outer over the same per-block row lists:
//   kv_kl     each chunk stages one block's K and K_idx rows in LDS; per 16 entry rows it
//             computes S_idx = Q_idx K_idx^T once on the matrix cores (one index head per
//             group, so the G heads of a row share it) and, per 16-row tile (16/G rows x
//             the G heads), S = Q K^T, the teacher weights t_j (the head mean), and per (row, slot)
//             the block's sums A = sum t ln t, B = sum t S^idx, T = sum t and the index
//             scores' (max, sum of 2^(z - max)) in log2 units.
//   kl_merge  per (b, r, row), one wave over the row's slots: L = A - B + lse_idx * T with
//             lse_idx = ln sum_j exp(S^idx_j) from the slots' (max, sum) pairs. (T is 1 up
//             to the rounding of the forward's lse; the loss keeps it as computed.)
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {
namespace {

// Stage rows [kb, kb+BS) of a row-major [*, D] array into LDS rows of ROWB bytes, 256
// threads. All loads are issued before the first LDS write; rows past n_k read row n_k - 1
// (their keys are masked later), so no load sits under a branch.
template <typename E, int D, int BS, int ROWB>
__device__ __forceinline__ void stage_rows(const E *src, long kb, int n_k, unsigned char *dst) {
  constexpr int PER_ROW = D * (int)sizeof(E) / 16, PIECES = BS * PER_ROW;
  constexpr int PT = (PIECES + 255) / 256;
  const int tid = threadIdx.x;
  const long last = (long)n_k - 1;
  u32x4 x[PT];
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int pc = min(tid + 256 * i, PIECES - 1);
    const long j = min(kb + pc / PER_ROW, last);
    x[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
        reinterpret_cast<const unsigned char *>(src + j * D) + (pc % PER_ROW) * 16));
  }
#pragma unroll
  for (int i = 0; i < PT; ++i) pin(x[i]);
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int pc = tid + 256 * i;
    if (PIECES % 256 == 0 || pc < PIECES)
      *reinterpret_cast<u32x4 *>(dst + (pc / PER_ROW) * ROWB + (pc % PER_ROW) * 16) = x[i];
  }
}

// Lane (l') of v inside each row of 16 lanes, l' named by the DPP control CTL.
template <int CTL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTL, 0xf, 0xf, false));
}
// Sum / max over the 16 lanes of a row: swaps within pairs and quads, then the half-row and
// row mirrors, each pairing every lane with one that holds the other half's partial.
__device__ __forceinline__ float sum16(float v) {
  v += dpp<0xb1>(v);   // quad_perm(1,0,3,2)
  v += dpp<0x4e>(v);   // quad_perm(2,3,0,1)
  v += dpp<0x141>(v);  // row_half_mirror
  return v + dpp<0x140>(v);  // row_mirror
}
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp<0xb1>(v));
  v = fmaxf(v, dpp<0x4e>(v));
  v = fmaxf(v, dpp<0x141>(v));
  return fmaxf(v, dpp<0x140>(v));
}

// S = Q K^T with the row-heads of a 16-row tile down the accumulator rows and the block's
// keys across the columns: lane (c16, g) holds key kt * 16 + c16 for row-heads m = 4g + i
// (row m >> log2g of the tile, head m & (G - 1)), i = 0..3. A row's G heads then sit in one
// lane (G <= 4) or in G / 4 lane groups (G = 8, 16), so the teacher's head mean is a few
// in-lane adds and at most two half-wave swaps. LG = min(log2g, 2): the value slots of one
// row in a lane are 1 << LG consecutive i; R4 = 4 >> LG rows per lane group.
template <typename E, int DH, int DI, int BS, int LG>
__global__ __launch_bounds__(256) void kv_kl(KvArgs a, KlArgs k, int log2g) {
  using F = typename Frag<E>::type;
  constexpr int ES = (int)sizeof(E);
  // Row pitches. A fragment read's 16 lanes of one LDS pass take rows 0-7 at 16-byte piece
  // p and rows 8-15 at piece p + 1: bf16 rows padded by 32 bytes put the two halves on the
  // even and odd 16-byte bank groups (16 bytes of padding left two lanes on one group).
  constexpr int PAD = ES == 2 ? 32 : 16;
  constexpr int KROW = DH * ES + PAD, IROW = DI * ES + PAD;
  // Index-score tile rows of BS + 4 floats: a write's lane groups (rows 4 g + i) start 16
  // banks apart.
  constexpr int SXR = BS + 4;
  constexpr int DC = DH / 32, DCI = DI / 32, KTN = BS / 16;
  constexpr int R4 = 4 >> LG;  // rows per lane group
  __shared__ __attribute__((aligned(16))) unsigned char s_k[BS * KROW];
  __shared__ __attribute__((aligned(16))) unsigned char s_ki[BS * IROW];
  __shared__ int32_t s_list[KV_CHUNK];
  // The list load below loops over a chunk's entries (any KV_CHUNK), but the tiles assume
  // the 256-thread workgroup that every KV_CHUNK up to 256 has been tested with.
  static_assert(KV_CHUNK <= 256, "kv_kl: chunks longer than the workgroup are untested");
  __shared__ float4 s_part[KV_CHUNK];  // the chunk's results, stored once per chunk: a store
  __shared__ float2 s_ml[KV_CHUNK];    // per tile would be waited for with the next loads
  __shared__ float s_sx[4][16][SXR];  // per wave: index scores of 16 entry rows x BS keys

  const long NB = (long)a.n_seg * a.batch * a.h_kv * a.n_blocks;
  const int n_chunks = a.coff[NB];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int G = 1 << log2g, QPT = 16 >> log2g;
  const int qi = c16 >> log2g, hd = c16 & (G - 1);  // the row-head this lane feeds to the A operand
  const E *q = reinterpret_cast<const E *>(a.q);
  const E *qx = reinterpret_cast<const E *>(k.q_idx);
  const float cs = a.scale_log2;                        // log2(e) / sqrt(d_h)
  const float ci = k.scale_idx * 1.44269504088896341f;  // log2(e) / sqrt(d_idx)
  const float inv_g = 1.f / (float)G;
  const bool writer_g = ((g * 4) & (G - 1)) == 0;  // first lane group of its rows

  __shared__ int s_next;
  for (int chunk = blockIdx.x; chunk < n_chunks; chunk = s_next) {  // uniform loop
    const long i = a.cmap[chunk];
    const int c = (int)(i % a.n_blocks);
    const long rsb = i / a.n_blocks;  // (r, seg, b) of the list
    const int b = (int)(rsb % a.batch);
    const int r = (int)(rsb / a.batch / a.n_seg);
    const int e0 = a.boff[i] + (chunk - a.coff[i]) * KV_CHUNK;
    const int n_e = min(e0 + KV_CHUNK, a.boff[i + 1]) - e0;
    const E *kp = reinterpret_cast<const E *>(a.k) + ((long)b * a.h_kv + r) * (long)a.cap * DH;
    const E *kip = reinterpret_cast<const E *>(k.k_idx) + (long)b * a.cap * DI;
    const long kb = (long)c * BS;
    const float *lse_r = k.lse + ((long)b * a.h_q + (long)r * G) * a.n_q;  // head r*G, row 0

    __syncthreads();  // the previous chunk is done with the LDS buffers and s_next
    if (tid == 0) s_next = claim_next(a.claim, n_chunks);  // chunks are claimed at run time
    for (int e = tid; e < n_e; e += 256) s_list[e] = a.list[e0 + e];  // any KV_CHUNK
    stage_rows<E, DH, BS, KROW>(kp, kb, a.n_k, s_k);
    stage_rows<E, DI, BS, IROW>(kip, kb, a.n_k, s_ki);
    __syncthreads();

    const int n_tiles = (n_e + QPT - 1) / QPT;
    // The next tile's inputs load while this one computes: q and q_idx of the row-head
    // this lane feeds, and the LSE of its four accumulator row-heads. Loads are
    // unconditional (lanes past the chunk's entries read entry 0's row and are masked), so
    // no load sits under a branch.
    struct TileIn {
      F q[DC];
      float lse[4];
    };
    // Tile row of accumulator slot ii: the slots of one row are 1 << LG consecutive i, so
    // for G >= 4 all four share row_slot(0) (written so the compiler sees it).
    auto row_slot = [&](int ii) { return (4 * g + ((ii >> LG) << LG)) >> log2g; };
    auto row_of = [&](int tt, int qm) {  // s_list entry of row qm of tile tt, or entry 0
      const int e = tt * QPT + qm;
      return s_list[(tt < n_tiles && e < n_e) ? e : 0];
    };
    auto load_tile = [&](int tt, TileIn &d) {
      const int t = row_of(tt, qi) >> 6;
      const E *src = q + (((long)b * a.h_q + r * G + hd) * a.n_q + t) * DH + g * 8;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) d.q[dc] = load_frag(src + dc * 32);
      const int t0 = row_of(tt, row_slot(0)) >> 6;  // slot rows: one lookup per row
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int tr = ((ii >> LG) << LG) == 0 ? t0 : row_of(tt, row_slot(ii)) >> 6;
        d.lse[ii] = lse_r[(long)((4 * g + ii) & (G - 1)) * a.n_q + tr];
      }
    };
    // Index scores of entry rows 16 gi .. 16 gi + 15 (the G tiles of row group gi) against
    // the block's keys, into this wave's LDS tile: s_sx[w][row][key]. The index query is
    // one head per group, so a tile's G heads share their row's scores and the product is
    // computed once per row instead of once per head.
    auto group_scores = [&](int gi) {
      const int e = gi * 16 + c16;
      const int t = s_list[e < n_e ? e : 0] >> 6;  // rows past the entries: entry 0, unused
      const E *srci = qx + (((long)b * a.h_kv + r) * a.n_q + t) * DI + g * 8;
      F aq[DCI];
#pragma unroll
      for (int dc = 0; dc < DCI; ++dc) aq[dc] = load_frag(srci + dc * 32);
      f32x4 sx[KTN];
#pragma unroll
      for (int kt = 0; kt < KTN; ++kt) sx[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < DCI; ++dc) {
        F kif[KTN];
#pragma unroll
        for (int kt = 0; kt < KTN; ++kt)
          kif[kt] = load_frag(reinterpret_cast<const E *>(s_ki + (kt * 16 + c16) * IROW +
                                                         (dc * 32 + g * 8) * ES));
#pragma unroll
        for (int kt = 0; kt < KTN; ++kt) sx[kt] = mfma_chunk(aq[dc], kif[kt], sx[kt]);
      }
#pragma unroll
      for (int kt = 0; kt < KTN; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_sx[w][4 * g + i][kt * 16 + c16] = sx[kt][i];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // wave-private tile: in-order LDS
    };
    // Wave w takes row groups w, w + 4, ... and the G tiles of each in turn.
    const int n_grp = (n_e + 15) / 16;
    int gi = w, u = 0, tt = w * G;
    TileIn cur, nxt;
    load_tile(tt, cur);
    while (gi < n_grp) {  // uniform over the wave
      if (u == 0) group_scores(gi);
      int gn = gi, un = u + 1;
      if (un == G || gn * G + un >= n_tiles) {
        gn = gi + 4;
        un = 0;
      }
      load_tile(gn * G + un, nxt);
      // an opaque zero offset keeps the compiler from hoisting the fragment reads below
      // out of the loop (kept in registers they would cost about a hundred VGPRs and a
      // third of the resident waves)
      int lds0 = 0;
      pin(lds0);
      // The KTN key tiles' products run as independent accumulation chains, one
      // d-chunk at a time (a chunk's fragments of every key tile are read first), so that
      // consecutive matrix-core operations do not wait on each other's results.
      f32x4 s[KTN];
#pragma unroll
      for (int kt = 0; kt < KTN; ++kt) s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        F kf[KTN];
#pragma unroll
        for (int kt = 0; kt < KTN; ++kt)
          kf[kt] = load_frag(reinterpret_cast<const E *>(s_k + lds0 + (kt * 16 + c16) * KROW +
                                                        (dc * 32 + g * 8) * ES));
#pragma unroll
        for (int kt = 0; kt < KTN; ++kt) s[kt] = mfma_chunk(cur.q[dc], kf[kt], s[kt]);
      }
      // this lane's index scores: row slot j's row of the group, key kt * 16 + c16
      float sv[KTN][R4];
#pragma unroll
      for (int j = 0; j < R4; ++j) {
        const int rho = u * QPT + row_slot(j << LG);
#pragma unroll
        for (int kt = 0; kt < KTN; ++kt) sv[kt][j] = s_sx[w][rho][kt * 16 + c16];
      }
      // per value slot: the key offset c16 of each tile is visible to its row iff <= lim
      int lim[4];
      float lse2[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        if (((ii >> LG) << LG) == ii) {  // first slot of its row
          const int qm = row_slot(ii);
          const bool valid = tt * QPT + qm < n_e;
          const long p = (long)a.q_start + (row_of(tt, qm) >> 6);
          lim[ii] = valid ? (int)min(p - kb, (long)BS - 1) : -1;
        } else {
          lim[ii] = lim[(ii >> LG) << LG];
        }
        lse2[ii] = cur.lse[ii] * 1.44269504088896341f;
      }
      float sa[R4], sb[R4], st[R4], zm[R4];
#pragma unroll
      for (int j = 0; j < R4; ++j) {
        sa[j] = 0.f;
        sb[j] = 0.f;
        st[j] = 0.f;
        zm[j] = -INFINITY;
      }
#pragma unroll
      for (int kt = 0; kt < KTN; ++kt) {
        const int key = kt * 16 + c16;
        float ph[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          ph[ii] = key <= lim[ii] ? __builtin_amdgcn_exp2f(fmaf(s[kt][ii], cs, -lse2[ii])) : 0.f;
        // the head mean of each row of this lane group
        float hs[R4];
#pragma unroll
        for (int j = 0; j < R4; ++j) {
          float v = 0.f;
#pragma unroll
          for (int u = 0; u < (1 << LG); ++u) v += ph[(j << LG) + u];
          hs[j] = v;
        }
        if constexpr (LG == 2) {  // G >= 4: one row per lane group, maybe across groups
          const float x8 = sum_xor16(hs[0]);
          const float x16 = sum_xor32(x8);
          hs[0] = log2g >= 4 ? x16 : (log2g == 3 ? x8 : hs[0]);
        }
#pragma unroll
        for (int j = 0; j < R4; ++j) {
          const int ii = j << LG;
          const float t = hs[j] * inv_g;
          const float sidx = sv[kt][j] * k.scale_idx;  // S^idx, natural units
          // t ln t, 0 at t = 0 (the clamp keeps the logarithm finite)
          sa[j] += t * (__builtin_amdgcn_logf(fmaxf(t, 1e-30f)) * 0.69314718055994531f);
          sb[j] += t * sidx;
          st[j] += t;
          zm[j] = key <= lim[ii] ? fmaxf(zm[j], sv[kt][j] * ci) : zm[j];
        }
      }
      // the tile's rows: totals over the 16 keys of each key tile (lanes of a row of 16)
#pragma unroll
      for (int j = 0; j < R4; ++j) {
        const int ii = j << LG;
        const float M = max16(zm[j]);
        float zl = 0.f;
#pragma unroll
        for (int kt = 0; kt < KTN; ++kt)
          zl += kt * 16 + c16 <= lim[ii] ? __builtin_amdgcn_exp2f(sv[kt][j] * ci - M) : 0.f;
        zl = sum16(zl);
        const float ta = sum16(sa[j]), tb = sum16(sb[j]), tt_ = sum16(st[j]);
        const int e = tt * QPT + row_slot(ii);
        if (c16 == 0 && writer_g && e < n_e) {
          s_part[e] = make_float4(ta, tb, tt_, 0.f);
          s_ml[e] = make_float2(M, zl);
        }
      }
      cur = nxt;
      gi = gn;
      u = un;
      tt = gn * G + un;
    }
    __syncthreads();
    for (int e = tid; e < n_e; e += 256) {
      const int ent = s_list[e];
      const long ps = (((long)b * a.h_kv + r) * a.n_q + (ent >> 6)) * a.top_k + (ent & 63);
      k.part[ps] = s_part[e];
      k.part_ml[ps] = s_ml[e];
    }
  }
}

// One wave per (b, r, row), a lane per slot (top_k <= 64): the row's partials are read
// as contiguous runs, then reduced across the wave.
__global__ __launch_bounds__(256) void kl_merge(KvArgs a, KlArgs k) {
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b, r, t)
  if (row >= (long)a.batch * a.h_kv * a.n_q) return;
  const int sl = threadIdx.x & 63;
  const int slc = min(sl, a.top_k - 1);  // lanes past top_k read the last slot, unused
  const int c = a.sel[row * a.top_k + slc];
  const float4 pa = k.part[row * a.top_k + slc];
  const float2 ml = k.part_ml[row * a.top_k + slc];
  const bool use = sl < a.top_k && c >= 0 && c < a.n_blocks;
  float A = use ? pa.x : 0.f, B = use ? pa.y : 0.f, T = use ? pa.z : 0.f;
  const bool has = use && ml.y > 0.f;
  float M = has ? ml.x : -INFINITY;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    A += __shfl_xor(A, o);
    B += __shfl_xor(B, o);
    T += __shfl_xor(T, o);
    M = fmaxf(M, __shfl_xor(M, o));
  }
  float L = has ? ml.y * __builtin_amdgcn_exp2f(ml.x - M) : 0.f;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
  if (sl == 0) {
    const float lse_idx = (M + __log2f(L)) * 0.69314718055994531f;
    k.kl[row] = A - B + lse_idx * T;
    if (k.lse_idx) k.lse_idx[row] = lse_idx;
  }
}

template <typename E, int DH, int DI, int BS, int LG>
hipError_t run_kl(const KvArgs &a, const KlArgs &k, int log2g, hipStream_t s) {
  static const int per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kv_kl<E, DH, DI, BS, LG>, 256, 0) !=
            hipSuccess || n < 1)
      n = 1;
    return n;
  }();
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const long NB = (long)a.n_seg * a.batch * a.h_kv * a.n_blocks;
  const long entries = (long)a.batch * a.h_kv * a.n_q * a.top_k;
  const long max_chunks = (entries + KV_CHUNK - 1) / KV_CHUNK + NB;
  // one round of the workgroups that fit on the device at once; chunks are claimed
  const unsigned grid = (unsigned)std::min(max_chunks, (long)per_cu * cus);
  KvArgs b = a;
  b.claim = a.cnt + 2 * NB;  // zeroed by the plan, after cnt and cursor
  hipLaunchKernelGGL((kv_kl<E, DH, DI, BS, LG>), dim3(grid), dim3(256), 0, s, b, k, log2g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long rows = (long)a.batch * a.h_kv * a.n_q;
  hipLaunchKernelGGL(kl_merge, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a, k);
  return hipGetLastError();
}

template <typename E, int DH, int DI, int BS>
hipError_t kl_groups(const KvArgs &a, const KlArgs &k, int lg, hipStream_t s) {
  if (lg == 0) return run_kl<E, DH, DI, BS, 0>(a, k, lg, s);
  if (lg == 1) return run_kl<E, DH, DI, BS, 1>(a, k, lg, s);
  return run_kl<E, DH, DI, BS, 2>(a, k, lg, s);
}

template <typename E, int DH>
hipError_t kl_dims(const KvArgs &a, const KlArgs &k, int d_idx, int lg, hipStream_t s) {
  if (d_idx == 32)
    return a.block_size == 32 ? kl_groups<E, DH, 32, 32>(a, k, lg, s) : kl_groups<E, DH, 32, 64>(a, k, lg, s);
  return a.block_size == 32 ? kl_groups<E, DH, 64, 32>(a, k, lg, s) : kl_groups<E, DH, 64, 64>(a, k, lg, s);
}

}  // namespace

hipError_t launch_index_kl(const KvArgs &a, const KlArgs &k, int dtype, int d_h, int d_idx,
                           hipStream_t s) {
  int lg = 0;
  while ((1 << lg) < a.h_q / a.h_kv) ++lg;
  if (dtype == 0)
    return d_h == 64 ? kl_dims<float, 64>(a, k, d_idx, lg, s) : kl_dims<float, 128>(a, k, d_idx, lg, s);
  return d_h == 64 ? kl_dims<bf16_t, 64>(a, k, d_idx, lg, s) : kl_dims<bf16_t, 128>(a, k, d_idx, lg, s);
}

}  // namespace msa
