// msa_attn.hip -- main branch for single-token decode: exact softmax attention over the
// selected blocks, split over the blocks and merged by log-sum-exp.
//
// Definition ("MiniMax-M3: MSA 技术报告速读", section 核心机制, main-branch equation):
// O^(h)_t = softmax(q_h k_T^T / sqrt(d_h)) v_T, T = visible tokens (j <= p) of the blocks
// the row's group selected; every head of a group shares the group's selection.
//
// A wave owns the G heads of one (sequence, group) (rows of a 16-row tile) and a fixed share
// of the selected blocks. Per block:
//   S^T = K_blk Q^T            (keys down the accumulator rows, one row per lane column)
//   online softmax in the log2 domain (per-lane row = lane % 16, reductions over 4 groups)
//   O^T += V_blk^T P^T         (P^T comes straight from the S^T accumulators: lane group g
//                               feeds keys {4g..4g+3} of two adjacent 16-key tiles, and the
//                               V^T fragment is read from LDS with the same key order)
// V is staged transposed in a wave-private LDS region; K fragments are read directly.
//
// Decode splits the selected blocks of one (sequence, group) over several waves, each
// writing (unnormalised O, running max, running sum); a second kernel merges them with
// log-sum-exp weights. The split is fixed on the host, so no atomics are used.
#include "msa_device.hpp"
#include "msa_internal.hpp"
#include "msa_select.hpp"

namespace msa {
namespace {

template <typename E, int DH, int BS>
struct VStage {
  static constexpr int ES = (int)sizeof(E);
  static constexpr int ROW = BS * ES + (ES == 2 ? 8 : 16);  // bytes per d-row of V^T
  static constexpr int BYTES = DH * ROW;
};

template <typename E, int DH, int BS>
struct RowState {
  static constexpr int DT = DH / 16;
  f32x4 o[DT];
  float m;  // running max, log2 units
  float l;  // running sum of 2^(z - m)
};

// V rows [kb, kb+BS) for one wave: loaded into registers first (so the loads overlap the
// score MFMAs), then written transposed into a wave-private LDS region vt[d][key].
template <typename E, int DH, int BS>
struct VRegs;
template <int DH, int BS>
struct VRegs<bf16_t, DH, BS> {  // key pairs packed into dwords
  static constexpr int PAIRS = BS / 2, SEGS = 64 / PAIRS, DSEG = DH / SEGS, PIECES = DSEG / 8;
  u32x4 a[PIECES], b[PIECES];
  __device__ __forceinline__ void load(const bf16_t *vp, long kb, int n_k) {
    const int lane = lane_id(), kp = lane % PAIRS, seg = lane / PAIRS;
    // keys past the end read the last key instead: their probabilities are 0
    const long j0 = min(kb + 2 * kp, (long)n_k - 1), j1 = min(kb + 2 * kp + 1, (long)n_k - 1);
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int d0 = seg * DSEG + i * 8;
      a[i] = *reinterpret_cast<const u32x4 *>(vp + j0 * DH + d0);
      b[i] = *reinterpret_cast<const u32x4 *>(vp + j1 * DH + d0);
    }
  }
  __device__ __forceinline__ void store_t(unsigned char *vt) const {
    constexpr int ROW = VStage<bf16_t, DH, BS>::ROW;
    const int lane = lane_id(), kp = lane % PAIRS, seg = lane / PAIRS;
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int d0 = seg * DSEG + i * 8;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = a[i][e], y = b[i][e];
        // element 2e is the low half, 2e+1 the high half of dword e
        *reinterpret_cast<uint32_t *>(vt + (d0 + 2 * e) * ROW + kp * 4) = (x & 0xffffu) | (y << 16);
        *reinterpret_cast<uint32_t *>(vt + (d0 + 2 * e + 1) * ROW + kp * 4) = (x >> 16) | (y & 0xffff0000u);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
};
template <int DH, int BS>
struct VRegs<float, DH, BS> {
  static constexpr int SEGS = 64 / BS, DSEG = DH / SEGS, PIECES = DSEG / 4;
  f32x4 a[PIECES];
  __device__ __forceinline__ void load(const float *vp, long kb, int n_k) {
    const int lane = lane_id(), key = lane % BS, seg = lane / BS;
    const long j = min(kb + key, (long)n_k - 1);  // past the end: probability 0
#pragma unroll
    for (int i = 0; i < PIECES; ++i)
      a[i] = *reinterpret_cast<const f32x4 *>(vp + j * DH + seg * DSEG + i * 4);
  }
  __device__ __forceinline__ void store_t(unsigned char *vt) const {
    constexpr int ROW = VStage<float, DH, BS>::ROW;
    const int lane = lane_id(), key = lane % BS, seg = lane / BS;
#pragma unroll
    for (int i = 0; i < PIECES; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<float *>(vt + (seg * DSEG + i * 4 + e) * ROW + key * 4) = a[i][e];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
};

// V^T fragment for d-row d and 32-key step ks: keys 32ks+4g+0..3 then 32ks+16+4g+0..3.
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
// P^T fragment for key step ks from the probability tiles 2ks and 2ks+1.
__device__ __forceinline__ bf16x8 pt_frag(f32x4 a, f32x4 b, const bf16_t *) {
  return __builtin_bit_cast(bf16x8, (u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                           pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])}));
}
__device__ __forceinline__ f32x8 pt_frag(f32x4 a, f32x4 b, const float *) {
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// One selected block for the wave's 16 rows. `active`: this lane's row takes part;
// p_row: its absolute position.
template <typename E, int DH, int BS>
__device__ __forceinline__ void attend_block(RowState<E, DH, BS> &st,
                                             const typename Frag<E>::type (&bq)[DH / 32],
                                             const E *kp, const E *vp, long kb, int n_k,
                                             bool active, long p_row, float scale_log2,
                                             unsigned char *vt) {
  using F = typename Frag<E>::type;
  constexpr int DC = DH / 32, KTN = BS / 16, DT = DH / 16;
  const int lane = lane_id(), g = lane >> 4, c16 = lane & 15;

  // All loads are unconditional (keys past the end read the last key and are masked below):
  // a load under a branch would make every MFMA wait for all loads issued before it.
  VRegs<E, DH, BS> vr;
  vr.load(vp, kb, n_k);  // in flight during the score MFMAs
  F ka[KTN][DC];
#pragma unroll
  for (int kt = 0; kt < KTN; ++kt) {
    const long j = min(kb + kt * 16 + c16, (long)n_k - 1);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) ka[kt][dc] = load_frag(kp + j * DH + dc * 32 + g * 8);
  }
  f32x4 s[KTN];
#pragma unroll
  for (int kt = 0; kt < KTN; ++kt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) acc = mfma_chunk(ka[kt][dc], bq[dc], acc);
    s[kt] = acc;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < KTN; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long j = kb + kt * 16 + g * 4 + i;
      const float z = (active && j <= p_row) ? s[kt][i] * scale_log2 : -INFINITY;
      s[kt][i] = z;
      mx = fmaxf(mx, z);
    }
  mx = max_groups(mx);
  const float m_new = fmaxf(st.m, mx);
  const float msub = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = exp2f(st.m - msub);
  float rs = 0.f;
#pragma unroll
  for (int kt = 0; kt < KTN; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pz = exp2f(s[kt][i] - msub);
      s[kt][i] = pz;
      rs += pz;
    }
  rs = sum_groups(rs);
  st.l = st.l * alpha + rs;
  st.m = m_new;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) st.o[dt] *= alpha;

  vr.store_t(vt);
  constexpr int ROW = VStage<E, DH, BS>::ROW;
#pragma unroll
  for (int ks = 0; ks < BS / 32; ++ks) {
    const F b = pt_frag(s[2 * ks], s[2 * ks + 1], kp);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const F a = vt_frag(vt + (dt * 16 + c16) * ROW, ks, g, kp);
      st.o[dt] = mfma_chunk(a, b, st.o[dt]);
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

template <typename E>
__device__ __forceinline__ void store4(E *dst, f32x4 v, float scale);
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t *dst, f32x4 v, float scale) {
  *reinterpret_cast<u32x2 *>(dst) =
      u32x2{pack_bf16x2(v[0] * scale, v[1] * scale), pack_bf16x2(v[2] * scale, v[3] * scale)};
}
template <>
__device__ __forceinline__ void store4<float>(float *dst, f32x4 v, float scale) {
  *reinterpret_cast<f32x4 *>(dst) = v * scale;
}

// Decode, split pass. Grid: x = groups of 4 waves over (b, r, split).
template <typename E, int DH, int BS>
__global__ __launch_bounds__(256) void attn_decode_split(AttnArgs a, int log2g) {
  using F = typename Frag<E>::type;
  using VS = VStage<E, DH, BS>;
  constexpr int DC = DH / 32, DT = DH / 16;
  __shared__ __attribute__((aligned(16))) unsigned char s_vt[4][VS::BYTES];

  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
  const int G = 1 << log2g, R = a.h_kv, S = a.splits;
  const long wid = (long)blockIdx.x * 4 + w;
  if (wid >= (long)a.batch * R * S) return;
  const int sp = (int)(wid % S);
  const int r = (int)((wid / S) % R);
  const int b = (int)(wid / ((long)S * R));
  const bool row_valid = c16 < G;
  const int h = r * G + (c16 & (G - 1));
  const long p_row = (long)a.q_start;

  const E *q = reinterpret_cast<const E *>(a.q);
  F bq[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
    bq[dc] = row_valid ? load_frag(q + ((long)b * a.h_q + h) * DH + dc * 32 + g * 8) : zero_frag(q);
  const long plane = ((long)b * R + r) * (long)a.cap * DH;
  const E *kp = reinterpret_cast<const E *>(a.k) + plane;
  const E *vp = reinterpret_cast<const E *>(a.v) + plane;
  const int32_t *selp = a.sel + ((long)b * R + r) * a.top_k;
  RowState<E, DH, BS> st;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
  const int e0 = sp * a.blocks_per_split, e1 = min(e0 + a.blocks_per_split, a.top_k);
  for (int e = e0; e < e1; ++e) {
    const int c = selp[e];
    if (c < 0) continue;  // wave-uniform
    attend_block<E, DH, BS>(st, bq, kp, vp, (long)c * BS, a.n_k, row_valid, p_row, a.scale_log2,
                            s_vt[w]);
  }
  if (row_valid) {
    const long pr = ((long)b * a.h_q + h) * S + sp;
    float *po = a.part_o + pr * DH;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4 *>(po + dt * 16 + g * 4) = st.o[dt];
    if (g == 0) {
      a.part_ml[pr * 2] = st.m;
      a.part_ml[pr * 2 + 1] = st.l;
    }
  }
}

// Decode, merge pass: one wave per (b, h); lanes cover d.
template <typename E, int DH>
__global__ __launch_bounds__(256) void attn_decode_merge(AttnArgs a) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long bh = (long)blockIdx.x * 4 + w;
  if (bh >= (long)a.batch * a.h_q) return;
  const int S = a.splits;  // <= 64
  const float2 mine = lane < S ? reinterpret_cast<const float2 *>(a.part_ml)[bh * S + lane]
                               : make_float2(-INFINITY, 0.f);
  float M = mine.y > 0.f ? mine.x : -INFINITY;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  const float wl = mine.y > 0.f ? __builtin_amdgcn_exp2f(mine.x - M) : 0.f;  // this split's weight
  float L = wl * mine.y;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
  constexpr int PER = DH / 64;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  const float *pbase = a.part_o + bh * S * DH + lane;
  for (int s0 = 0; s0 < S; s0 += 8) {  // eight splits' loads in flight together
    float wv[8], pv[8][PER];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sp = s0 + u;
      wv[u] = __shfl(wl, sp & 63);  // 0 for splits past S (their lanes hold weight 0)
      // unconditional loads (every split's partial is written, zeros if it saw no key);
      // splits past S re-read the last one and are weighted 0
      const int spc = min(sp, S - 1);
#pragma unroll
      for (int i = 0; i < PER; ++i) pv[u][i] = pbase[spc * DH + 64 * i];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] += wv[u] * pv[u][i];
  }
  const float inv = 1.f / L;
  E *o = reinterpret_cast<E *>(a.o) + bh * DH;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const float x = acc[i] * inv;
    if constexpr (sizeof(E) == 2) {
      reinterpret_cast<uint16_t *>(o)[lane + 64 * i] = (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu);
    } else {
      reinterpret_cast<float *>(o)[lane + 64 * i] = x;
    }
  }
  if (a.lse && lane == 0) a.lse[bh] = (M + __log2f(L)) * 0.69314718055994531f;
}

constexpr int cmax(int x, int y) { return x > y ? x : y; }

template <typename E>
__device__ __forceinline__ void store1(E *dst, float x) {
  if constexpr (sizeof(E) == 2)
    *reinterpret_cast<uint16_t *>(dst) = (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu);
  else
    *reinterpret_cast<float *>(dst) = x;
}

// Decode, everything after the index kernel in one launch. Grid: x = (b, r) pair * subs +
// sub; four waves.
//   1. Every workgroup of a pair merges the pair's per-range winners into the selection (the
//      two stages of the wide merge; sub 0 also writes sel). Repeating this small merge in
//      each of the pair's few workgroups costs less than a launch between them.
//   2. Wave w attends the selected blocks e0 + w, e0 + w + 4, ... of the sub's share
//      [e0, e1), one online softmax per wave.
//   3. The four waves' (o, m, l) are merged in LDS into the sub's partial.
//   4. With one workgroup per pair it writes o and lse. Otherwise each workgroup stores its
//      partial and bumps the pair's device-scope counter; the last to arrive merges the
//      pair's partials in sub order. The counters are cleared by the index kernel of the
//      same step, so a step needs no clearing launch of its own.
template <typename E, int DH, int BS>
__global__ __launch_bounds__(256) void decode_finish(AttnArgs a, FinishArgs f, int log2g) {
  using F = typename Frag<E>::type;
  using VS = VStage<E, DH, BS>;
  constexpr int DC = DH / 32, DT = DH / 16;
  constexpr int SEL_BYTES = 8 * SELECT_LDS * 4 + 2 * 256 * 4;  // lk, li per wave; w_key, w_idx
  // per wave: o[16][MROW], (m, l)[16]; rows of DH + 4 floats, so the 16-byte stores of 8
  // consecutive lanes (8 rows) start on different bank groups (DH floats put them on one)
  constexpr int MROW = DH + 4;
  constexpr int MRG_BYTES = 4 * 16 * MROW * 4 + 4 * 16 * 8;
  constexpr int BUF = cmax(4 * VS::BYTES, cmax(SEL_BYTES, MRG_BYTES));
  __shared__ __attribute__((aligned(16))) unsigned char s_buf[BUF];
  __shared__ int32_t s_sel[64];
  __shared__ int s_last;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int G = 1 << log2g, R = a.h_kv, k = a.top_k, m = k - 1;
  const int pair = blockIdx.x / f.subs, sub = blockIdx.x % f.subs;
  const int b = pair / R, r = pair % R;
  const long p = (long)a.q_start;
  const int local = (int)(p / a.block_size);

  // the query rows (G heads of the pair, rows of a 16-row tile) load while the selection runs
  const bool row_valid = c16 < G;
  const int h = r * G + (c16 & (G - 1));
  const E *q = reinterpret_cast<const E *>(a.q);
  F bq[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
    bq[dc] = load_frag(q + ((long)b * a.h_q + h) * DH + dc * 32 + g * 8);  // rows >= G: masked

  // 1. selection
  if (local + 1 <= k || m == 0) {  // sees k blocks or fewer, or k == 1 (uniform)
    if (tid < k) s_sel[tid] = local + 1 <= k ? (tid <= local ? tid : -1) : (tid == 0 ? local : -1);
  } else {
    uint32_t *lk = reinterpret_cast<uint32_t *>(s_buf) + w * SELECT_LDS;
    int32_t *li = reinterpret_cast<int32_t *>(s_buf) + (4 + w) * SELECT_LDS;
    uint32_t *w_key = reinterpret_cast<uint32_t *>(s_buf) + 8 * SELECT_LDS;
    int32_t *w_idx = reinterpret_cast<int32_t *>(s_buf) + 8 * SELECT_LDS + 256;
    const int nch = (local + SEL_NBLK - 1) / SEL_NBLK;  // ranges holding candidates
    const long base = (long)pair * f.n_wg * m;
    wide_stage1<4>(f.cand_key + base, f.cand_idx + base, nch * m, m, w, lk, li, w_key, w_idx);
    __syncthreads();
    if (w == 0) {
      wide_stage2<4>(m, w_key, w_idx, lk, li, [&](int j, int32_t c) { s_sel[j] = c; });
      if (lane == 0) s_sel[m] = local;
    }
  }
  __syncthreads();
  if (sub == 0 && tid < k) f.sel[(long)pair * k + tid] = s_sel[tid];

  // 2. attention over the sub's share of the selected blocks
  const long plane = ((long)b * R + r) * (long)a.cap * DH;
  const E *kp = reinterpret_cast<const E *>(a.k) + plane;
  const E *vp = reinterpret_cast<const E *>(a.v) + plane;
  RowState<E, DH, BS> st;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
  const int per = (k + f.subs - 1) / f.subs;
  const int e0 = sub * per, e1 = min(e0 + per, k);
  for (int e = e0 + w; e < e1; e += 4) {
    const int c = s_sel[e];
    if (c < 0) continue;  // wave-uniform
    attend_block<E, DH, BS>(st, bq, kp, vp, (long)c * BS, a.n_k, row_valid, p, a.scale_log2,
                            s_buf + w * VS::BYTES);
  }

  // 3. the four waves' partials, merged in LDS (the V^T regions are free once all are done)
  __syncthreads();
  float *mo = reinterpret_cast<float *>(s_buf);                         // [4][16][MROW]
  float2 *mml = reinterpret_cast<float2 *>(s_buf + 4 * 16 * MROW * 4);  // [4][16]
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    *reinterpret_cast<f32x4 *>(mo + (w * 16 + c16) * MROW + dt * 16 + g * 4) = st.o[dt];
  if (g == 0) mml[w * 16 + c16] = make_float2(st.m, st.l);
  __syncthreads();
  E *o = reinterpret_cast<E *>(a.o);
  const int n_out = G * DH;
  for (int x = tid; x < n_out; x += 256) {
    const int hh = x / DH, d = x % DH;
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float2 ml = mml[u * 16 + hh];
      if (ml.y > 0.f) M = fmaxf(M, ml.x);
    }
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float2 ml = mml[u * 16 + hh];
      if (ml.y > 0.f) {
        const float wt = __builtin_amdgcn_exp2f(ml.x - M);
        L += wt * ml.y;
        O += wt * mo[(u * 16 + hh) * MROW + d];
      }
    }
    const long bh = (long)b * a.h_q + r * G + hh;
    if (f.subs == 1) {  // the whole selection: final output (the local block makes L > 0)
      store1(o + bh * DH + d, O / L);
      if (a.lse && d == 0) a.lse[bh] = (M + __log2f(L)) * 0.69314718055994531f;
    } else {
      const long sp = ((long)pair * f.subs + sub) * G + hh;
      a.part_o[sp * DH + d] = O;
      if (d == 0) {
        a.part_ml[sp * 2] = M;
        a.part_ml[sp * 2 + 1] = L;
      }
    }
  }
  if (f.subs == 1) return;

  // 4. the last workgroup of the pair to arrive merges the subs' partials. One thread per
  // workgroup fences: a device-scope fence writes back (release) or invalidates (acquire)
  // the XCD's L2, so one per thread would repeat that 256 times. Each wave first waits for
  // its own partial stores to complete (the workgroup barrier alone does not wait for
  // global stores), so that they are in L2 when thread 0's release writes it back; the
  // barrier after the count orders the other threads' loads after what thread 0 acquires.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    __threadfence();  // the workgroup's partials are visible device-wide before its count
    s_last = atomicAdd(f.cnt + pair, 1) == f.subs - 1;
    if (s_last) __threadfence();  // the other workgroups' partials are read after their counts
  }
  __syncthreads();
  if (!s_last) return;
  // Four consecutive outputs of one head per thread; every sub's (m, l) and partial of them
  // load together (subs <= FINISH_MAX_SUBS; past subs the last one is re-read and weighted 0).
  const float2 *pml = reinterpret_cast<const float2 *>(a.part_ml);
  for (int x4 = tid; x4 < n_out / 4; x4 += 256) {
    const int hh = (x4 * 4) / DH, d0 = (x4 * 4) % DH;
    const long sp0 = (long)pair * f.subs * G + hh;  // sub u's partial: sp0 + u * G
    float2 ml[FINISH_MAX_SUBS];
    f32x4 po[FINISH_MAX_SUBS];
#pragma unroll
    for (int u = 0; u < FINISH_MAX_SUBS; ++u) {
      const long sp = sp0 + (long)min(u, f.subs - 1) * G;
      ml[u] = pml[sp];
      po[u] = *reinterpret_cast<const f32x4 *>(a.part_o + sp * DH + d0);
    }
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < FINISH_MAX_SUBS; ++u)
      if (u < f.subs && ml[u].y > 0.f) M = fmaxf(M, ml[u].x);
    float L = 0.f;
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < FINISH_MAX_SUBS; ++u) {
      const float wt = (u < f.subs && ml[u].y > 0.f) ? __builtin_amdgcn_exp2f(ml[u].x - M) : 0.f;
      L += wt * ml[u].y;
      O += wt * po[u];
    }
    const long bh = (long)b * a.h_q + r * G + hh;
    const float inv = 1.f / L;
#pragma unroll
    for (int e = 0; e < 4; ++e) store1(o + bh * DH + d0 + e, O[e] * inv);
    if (a.lse && d0 == 0) a.lse[bh] = (M + __log2f(L)) * 0.69314718055994531f;
  }
}

template <typename E, int DH>
hipError_t finish_t(const AttnArgs &a, const FinishArgs &f, int bs, int log2g, hipStream_t s) {
  const dim3 grid((unsigned)((long)a.batch * a.h_kv * f.subs));
  if (bs == 32)
    hipLaunchKernelGGL((decode_finish<E, DH, 32>), grid, dim3(256), 0, s, a, f, log2g);
  else
    hipLaunchKernelGGL((decode_finish<E, DH, 64>), grid, dim3(256), 0, s, a, f, log2g);
  return hipGetLastError();
}

template <typename E, int DH>
hipError_t decode_t(const AttnArgs &a, int bs, int log2g, hipStream_t s) {
  const long waves = (long)a.batch * a.h_kv * a.splits;
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (bs == 32)
    hipLaunchKernelGGL((attn_decode_split<E, DH, 32>), grid, dim3(256), 0, s, a, log2g);
  else
    hipLaunchKernelGGL((attn_decode_split<E, DH, 64>), grid, dim3(256), 0, s, a, log2g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long mw = (long)a.batch * a.h_q;
  hipLaunchKernelGGL((attn_decode_merge<E, DH>), dim3((unsigned)((mw + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

int ilog2(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

}  // namespace

hipError_t launch_decode_finish(const AttnArgs &a, const FinishArgs &f, int dtype, int d_h,
                                hipStream_t s) {
  const int lg = ilog2(a.h_q / a.h_kv);
  if (dtype == 0) return d_h == 64 ? finish_t<float, 64>(a, f, a.block_size, lg, s)
                                   : finish_t<float, 128>(a, f, a.block_size, lg, s);
  return d_h == 64 ? finish_t<bf16_t, 64>(a, f, a.block_size, lg, s)
                   : finish_t<bf16_t, 128>(a, f, a.block_size, lg, s);
}

hipError_t launch_attn_decode(const AttnArgs &a, int dtype, int d_h, hipStream_t s) {
  const int lg = ilog2(a.h_q / a.h_kv);
  if (dtype == 0) return d_h == 64 ? decode_t<float, 64>(a, a.block_size, lg, s)
                                   : decode_t<float, 128>(a, a.block_size, lg, s);
  return d_h == 64 ? decode_t<bf16_t, 64>(a, a.block_size, lg, s)
                   : decode_t<bf16_t, 128>(a, a.block_size, lg, s);
}

}  // namespace msa
