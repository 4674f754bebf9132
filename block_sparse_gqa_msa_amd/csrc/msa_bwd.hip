// msa_bwd.hip -- gradients of the main branch (dq, dk, dv) for a fixed block selection.
//
// The forward is the main-branch equation of "MiniMax-M3: MSA 技术报告速读" (section
// 核心机制); the training section of the same page detaches the index branch, so the
// selection is a constant here and only q, k and v receive gradients. For row t, head h
// and the visible tokens T of the selected blocks, with P_j = exp(q . k_j / sqrt(d_h) - lse)
// and D = sum_d dO_d O_d (which equals sum_j P_j dP_j):
//   dP_j = dO . v_j,   dS_j = P_j (dP_j - D),
//   dv_j += P_j dO,    dk_j += dS_j q / sqrt(d_h),   dq = sum_j dS_j k_j / sqrt(d_h).
// Organised KV-block-outer over the prefill's per-block row lists (the page's Kernel
// section gathers the rows that chose a block so a staged block serves all of them):
//   bwd_rowdot  D per (b, h, t) from o and dout.
//   kv_bwd      persistent over runs of RUN consecutive chunks, claimed at run time. A
//               chunk's block is split over BS / 16 waves, 16 keys each. Per 32-row-head
//               tile (32 / G rows x the G heads) every wave computes S = Q K_w^T and
//               dP = dO V_w^T on the matrix cores with the row-heads down the accumulator
//               rows; the accumulator layout is then directly the A operand of
//               dV_w += P^T dO and dK_w += dS^T Q, whose B operands are the staged Q and
//               dO tiles read transposed (bf16: in place, with the matrix cores'
//               transposing LDS read; fp32: from transposed copies). dS goes to LDS, and each wave
//               computes dq for its slice of d over the whole block, written as one partial
//               per (row, slot, head). dK_w and dV_w stay in registers while a run stays on
//               one list and are written as one fp32 partial per (run, list) segment.
//   dq_merge    dq = the sum of the row's partials in slot order.
//   dkv_reduce  per (b, r, block), the sum of its segments' partials in chunk order.
// No float atomics reach memory. dq does not depend on the order of a list's entries; dk
// and dv sum a chunk's rows in list order, which the list build's integer atomics set, so
// they can differ between calls in the last bits.
#include "msa_device.hpp"
#include "msa_internal.hpp"

#include <algorithm>
#include <cmath>

namespace msa {
namespace {

constexpr int CHUNK = KV_CHUNK;
constexpr int TR = 32;  // row-heads per tile

// List index of (b, r, row segment, block), as the list build keys it.
__device__ __forceinline__ long bwd_list_index(const KvArgs &a, int b, int r, int seg, int c) {
  return (((long)r * a.n_seg + seg) * a.batch + b) * a.n_blocks + c;
}

// ---------------------------------------------------------------- D = rowsum(dO * O)

// DH / 8 consecutive threads per (b, h, t) row, 8 elements each.
template <typename E, int DH>
__global__ __launch_bounds__(256) void bwd_rowdot(const E *o, const E *dout, float *dsum, long rows) {
  constexpr int LPR = DH / 8;
  const long gl = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = gl / LPR;
  const int j = (int)(gl % LPR);
  float acc = 0.f;
  if (row < rows) {
    const long off = row * DH + j * 8;
    if constexpr (sizeof(E) == 2) {
      const u32x4 x = *reinterpret_cast<const u32x4 *>(o + off);
      const u32x4 y = *reinterpret_cast<const u32x4 *>(dout + off);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(__uint_as_float(x[e] << 16), __uint_as_float(y[e] << 16), acc);
        acc = fmaf(__uint_as_float(x[e] & 0xffff0000u), __uint_as_float(y[e] & 0xffff0000u), acc);
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4 x = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(o) + off + 4 * h);
        const f32x4 y = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(dout) + off + 4 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = fmaf(x[e], y[e], acc);
      }
    }
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (row < rows && j == 0) dsum[row] = acc;
}

// ---------------------------------------------------------------- per-block gradients

template <typename E, int DH, int BS>
struct BwdLds {
  static constexpr int ES = (int)sizeof(E);
  static constexpr int NW = BS / 16;                 // waves: 16 keys each
  static constexpr int NT = 64 * NW;                 // threads
  static constexpr int DSL = DH / NW;                // dq columns per wave
  static constexpr int PE = 16 / ES;                 // elements per 16-byte piece
  // Row pitches. A matrix-core fragment read puts rows 0-7 at 16-byte piece p and rows
  // 8-15 at piece p + 1 in one 16-lane group of the LDS; bf16 rows of 256 or 128 bytes
  // padded by 32 bytes place the two halves on even and odd 16-byte bank groups, with
  // addresses that stay linear (16-byte padding collided there). Other shapes keep 16.
  static constexpr bool P32Q = ES == 2 && DH * ES == 256;
  static constexpr bool P32S = ES == 2 && BS * ES == 128;
  static constexpr int QPIECES = DH * ES / 16;             // 16-byte pieces per Q, dO row
  static constexpr int QROW = DH * ES + (P32Q ? 32 : 16);  // Q, dO row-major rows
  static constexpr int TROW = TR * ES + 16;               // fp32 Q^T, dO^T rows (one per d)
  static constexpr int SROW = BS * ES + (P32S ? 32 : 16);  // dS rows, K^T rows
  static constexpr int OROW = DSL * ES + 16;              // per-wave dq staging rows
  static constexpr int NTASK = 16 * (DH / PE);       // (row pair, piece) tasks per tensor
  static constexpr int TPT = 2 * NTASK / NT;         // staging tasks per thread (Q and dO)
  static_assert(NT == 4 * BS && 2 * NTASK % NT == 0, "staging tasks must divide evenly");
};

// B side of dV += P^T dO and dK += dS^T Q, bf16: the 8 K-elements of a 32-wide chunk whose
// A side comes from two accumulator tiles are row-heads 4g + 0..3, then 16 + 4g + 0..3,
// for column d0 + lane % 16. They are read transposed straight from the row-major tile with
// ds_read_b64_tr_b16: in each 16-lane group, lanes 4s .. 4s + 3 give the addresses of the
// four 4-element pieces of row s (columns d0 .. d0 + 15), and lane i receives element i of
// the group's four rows. With 288-byte rows the 8 rows of a 32-lane group sit on distinct
// pairs of 16-byte bank groups.
template <typename L>
__device__ __forceinline__ bf16x8 tr_frag_rm(const unsigned char *tile, int d0, int g, int lane) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef short v8s __attribute__((ext_vector_type(8)));
  typedef __attribute__((address_space(3))) v4s *lds_v4s;
  const int s = (lane & 15) >> 2, j = lane & 3;
  unsigned char *p = const_cast<unsigned char *>(tile) + (4 * g + s) * L::QROW + (d0 + 4 * j) * 2;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p + 16 * L::QROW));
  return __builtin_bit_cast(bf16x8, (v8s{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}));
}
// fp32: the same 8 K-elements from transposed staging row d (one row per column).
__device__ __forceinline__ f32x8 tr_frag(const unsigned char *row, int g) {
  const f32x4 lo = *reinterpret_cast<const f32x4 *>(row + (4 * g) * 4);
  const f32x4 hi = *reinterpret_cast<const f32x4 *>(row + (16 + 4 * g) * 4);
  return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// Two accumulator tiles' four values each as the A side of the same chunk.
__device__ __forceinline__ bf16x8 acc_frag(f32x4 a, f32x4 b, const bf16_t *) {
  return __builtin_bit_cast(bf16x8, (u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                           pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])}));
}
__device__ __forceinline__ f32x8 acc_frag(f32x4 a, f32x4 b, const float *) {
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ void put1(unsigned char *p, float v, const bf16_t *) {
  *reinterpret_cast<uint16_t *>(p) = (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu);
}
__device__ __forceinline__ void put1(unsigned char *p, float v, const float *) {
  *reinterpret_cast<float *>(p) = v;
}

// Stage K^T of block rows [kb, kb + BS) (one LDS row of BS keys per d), NT threads. Rows
// past n_k read row n_k - 1 (their keys are masked, so their dS are 0).
template <typename E, int DH, int BS, int NT>
__device__ __forceinline__ void stage_kt(const E *kp, long kb, int n_k, unsigned char *kt) {
  using L = BwdLds<E, DH, BS>;
  const int tid = threadIdx.x;
  const long last = (long)n_k - 1;
  if constexpr (L::ES == 2) {
    constexpr int PAIRS = BS / 2, PIECES = PAIRS * (DH / 8), PT = (PIECES + NT - 1) / NT;
    u32x4 x[PT], y[PT];
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int pc = min(tid + NT * i, PIECES - 1);
      const int kpair = pc % PAIRS, d0 = (pc / PAIRS) * 8;
      const long j0 = min(kb + 2 * kpair, last), j1 = min(kb + 2 * kpair + 1, last);
      x[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kp + j0 * DH + d0));
      y[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kp + j1 * DH + d0));
    }
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      pin(x[i]);
      pin(y[i]);
    }
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int pc = tid + NT * i;
      if (PIECES % NT == 0 || pc < PIECES) {
        const int kpair = pc % PAIRS, d0 = (pc / PAIRS) * 8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t a = x[i][e], b = y[i][e];
          *reinterpret_cast<uint32_t *>(kt + (d0 + 2 * e) * L::SROW + kpair * 4) = (a & 0xffffu) | (b << 16);
          *reinterpret_cast<uint32_t *>(kt + (d0 + 2 * e + 1) * L::SROW + kpair * 4) = (a >> 16) | (b & 0xffff0000u);
        }
      }
    }
  } else {
    constexpr int PIECES = BS * (DH / 4), PT = (PIECES + NT - 1) / NT;
    f32x4 x[PT];
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int pc = min(tid + NT * i, PIECES - 1);
      const long j = min(kb + pc % BS, last);
      x[i] = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(kp) + j * DH + (pc / BS) * 4);
    }
#pragma unroll
    for (int i = 0; i < PT; ++i) pin(x[i]);
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int pc = tid + NT * i;
      if (PIECES % NT == 0 || pc < PIECES) {
        const int key = pc % BS, d0 = (pc / BS) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) *reinterpret_cast<float *>(kt + (d0 + e) * L::SROW + key * 4) = x[i][e];
      }
    }
  }
}

struct BwdArgs {
  const void *dout;   // [B, H, n_q, DH]
  const float *lse;   // [B, H, n_q] natural log, from the forward
  const float *dsum;  // [B, H, n_q] D = rowsum(dO * O)
  float *dkv;         // [slots][2][BS][DH] fp32 segment partials (dK, then dV)
  void *dq, *dk, *dv;
  float scale;        // 1 / sqrt(d_h)
  int run;            // chunks per run
  long run_slots;     // slot index of list i's first segment when it starts inside a run
};

template <typename E, int DH, int BS>
__global__ __launch_bounds__(4 * BS) void kv_bwd(KvArgs a, BwdArgs w, int log2g) {
  using F = typename Frag<E>::type;
  using L = BwdLds<E, DH, BS>;
  constexpr int NW = L::NW, NT = L::NT, DSL = L::DSL, DC = DH / 32, DT = DH / 16;
  constexpr int QN = DSL / 16, KS = BS / 32;
  __shared__ __attribute__((aligned(16))) unsigned char s_q[TR * L::QROW];
  __shared__ __attribute__((aligned(16))) unsigned char s_do[TR * L::QROW];
  // transposed copies: fp32 only (bf16 reads the row-major tiles transposed)
  __shared__ __attribute__((aligned(16))) unsigned char s_qt[L::ES == 2 ? 16 : DH * L::TROW];
  __shared__ __attribute__((aligned(16))) unsigned char s_dot[L::ES == 2 ? 16 : DH * L::TROW];
  __shared__ __attribute__((aligned(16))) unsigned char s_ds[TR * L::SROW];
  __shared__ __attribute__((aligned(16))) unsigned char s_kt[DH * L::SROW];
  __shared__ __attribute__((aligned(16))) unsigned char s_o[NW][TR * L::OROW];
  __shared__ __attribute__((aligned(16))) float s_lse2[TR];
  __shared__ __attribute__((aligned(16))) float s_dd[TR];
  __shared__ __attribute__((aligned(16))) int s_pos[TR];
  __shared__ int32_t s_list[CHUNK];

  const long NB = (long)a.n_seg * a.batch * a.h_kv * a.n_blocks;
  const int n_chunks = a.coff[NB];
  const int n_runs = (n_chunks + w.run - 1) / w.run;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int G = 1 << log2g, RPT = TR >> log2g;
  const E *qg = reinterpret_cast<const E *>(a.q);
  const E *dog = reinterpret_cast<const E *>(w.dout);
  const E *tagp = nullptr;
  const float cs = a.scale_log2, dscale = w.scale;
  constexpr float LOG2E = 1.4426950408889634f;

  __shared__ int s_next;
  for (int run = blockIdx.x; run < n_runs; run = s_next) {  // uniform loop
    __syncthreads();  // every thread has read s_next for this run
    if (tid == 0) s_next = claim_next(a.claim, n_runs);  // runs are claimed at run time
    const int c0 = run * w.run, c1 = min(c0 + w.run, n_chunks);
    long cur = -1;
    int seg_first = 0, b = 0, r = 0;
    long kb = 0;
    F kq[DC], vq[DC], ktf[QN][KS];
    f32x4 dk[DT], dv[DT];

    auto flush = [&]() {
      const long slot = seg_first % w.run == 0 ? seg_first / w.run : w.run_slots + cur;
      float *base = w.dkv + slot * (2L * BS * DH);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const long off = (long)(16 * wv + 4 * g + i) * DH + 16 * dt + c16;
          base[off] = dk[dt][i];
          base[(long)BS * DH + off] = dv[dt][i];
        }
    };

    for (int chunk = c0; chunk < c1; ++chunk) {
      const long i = a.cmap[chunk];
      if (i != cur) {  // a new list: new block, fresh accumulators
        if (cur >= 0) flush();
        cur = i;
        seg_first = chunk;
        const int c = (int)(i % a.n_blocks);
        const long rsb = i / a.n_blocks;
        b = (int)(rsb % a.batch);
        r = (int)(rsb / a.batch / a.n_seg);
        kb = (long)c * BS;
        const long plane = ((long)b * a.h_kv + r) * (long)a.cap * DH;
        const E *kp = reinterpret_cast<const E *>(a.k) + plane;
        const E *vp = reinterpret_cast<const E *>(a.v) + plane;
        const long krow = min(kb + 16 * wv + c16, (long)a.n_k - 1);
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          kq[dc] = load_frag(kp + krow * DH + dc * 32 + g * 8);
          vq[dc] = load_frag(vp + krow * DH + dc * 32 + g * 8);
        }
        __syncthreads();  // the previous list's K^T reads are done
        stage_kt<E, DH, BS, NT>(kp, kb, a.n_k, s_kt);
        __syncthreads();
#pragma unroll
        for (int nt = 0; nt < QN; ++nt)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            ktf[nt][ks] = load_frag(reinterpret_cast<const E *>(
                s_kt + (wv * DSL + nt * 16 + c16) * L::SROW + (ks * 32 + g * 8) * L::ES));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          dk[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
          dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      const int e0 = a.boff[cur] + (chunk - a.coff[cur]) * CHUNK;
      const int n_e = min(e0 + CHUNK, a.boff[cur + 1]) - e0;
      __syncthreads();  // the previous chunk is done with s_list
      for (int e = tid; e < n_e; e += NT) s_list[e] = a.list[e0 + e];  // NT may be < CHUNK
      __syncthreads();
      const int n_tiles = (n_e + RPT - 1) / RPT;
      const long head0 = (long)b * a.h_q + (long)r * G;

      // Tile staging: every load is unconditional (rows past the chunk's entries read the
      // first entry's row and are masked) so the next tile's loads stay in flight.
      u32x4 px[L::TPT][2];
      float plse = 0.f, pd = 0.f;
      int ppos = -1;
      bool pok = false;
      auto load_tile = [&](int tt) {
#pragma unroll
        for (int j = 0; j < L::TPT; ++j) {
          const int task = tid + NT * j;
          const int tensor = task / L::NTASK, tk = task % L::NTASK;
          const int p = tk / (DH / L::PE), dg = tk % (DH / L::PE);
          const E *src = tensor ? dog : qg;
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int m = 2 * p + h2;
            const int e = tt * RPT + (m >> log2g);
            const int t = s_list[e < n_e ? e : 0] >> 6;
            px[j][h2] = *reinterpret_cast<const u32x4 *>(
                src + ((head0 + (m & (G - 1))) * a.n_q + t) * DH + dg * L::PE);
          }
        }
        {  // every thread loads (threads past TR repeat a row): no branch around the loads
          const int mrow = tid & (TR - 1);
          const int e = tt * RPT + (mrow >> log2g);
          pok = e < n_e;
          const int t = s_list[pok ? e : 0] >> 6;
          const long row = (head0 + (mrow & (G - 1))) * a.n_q + t;
          plse = w.lse[row];
          pd = w.dsum[row];
          ppos = a.q_start + t;
        }
      };
      auto write_tile = [&]() {
#pragma unroll
        for (int j = 0; j < L::TPT; ++j) {
          const int task = tid + NT * j;
          const int tensor = task / L::NTASK, tk = task % L::NTASK;
          const int p = tk / (DH / L::PE), dg = tk % (DH / L::PE);
          unsigned char *rm = tensor ? s_do : s_q;
          *reinterpret_cast<u32x4 *>(rm + (2 * p) * L::QROW + dg * 16) = px[j][0];
          *reinterpret_cast<u32x4 *>(rm + (2 * p + 1) * L::QROW + dg * 16) = px[j][1];
          if constexpr (L::ES == 4) {  // fp32: transposed copy (one row per d)
            unsigned char *tr = tensor ? s_dot : s_qt;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              *reinterpret_cast<u32x2 *>(tr + (dg * 4 + e) * L::TROW + p * 8) = u32x2{px[j][0][e], px[j][1][e]};
          }
        }
        if (tid < TR) {
          s_lse2[tid] = pok ? plse * LOG2E : INFINITY;
          s_dd[tid] = pok ? pd : 0.f;
          s_pos[tid] = pok ? ppos : -1;
        }
      };

      // Tile tt + 1 is staged after tile tt's dq stores, and its loads were issued after
      // tile tt - 1's: at every staging point the same stores are younger than the loads
      // it waits for, so the wait counts them and leaves them in flight. (Staging at the
      // top of the loop would merge with the loop entry, where nothing follows the loads,
      // into a wait for everything.)
      load_tile(0);
      write_tile();
      load_tile(min(1, n_tiles - 1));
      __syncthreads();
      for (int tt = 0; tt < n_tiles; ++tt) {

        // S and dP for this wave's 16 keys, row-heads 16 mt + 4 g + i down the rows
        f32x4 s[2], dp[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          f32x4 as = {0.f, 0.f, 0.f, 0.f}, ad = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int dc = 0; dc < DC; ++dc) {
            const F fq = load_frag(reinterpret_cast<const E *>(s_q + (mt * 16 + c16) * L::QROW + (dc * 32 + g * 8) * L::ES));
            const F fo = load_frag(reinterpret_cast<const E *>(s_do + (mt * 16 + c16) * L::QROW + (dc * 32 + g * 8) * L::ES));
            as = mfma_chunk(fq, kq[dc], as);
            ad = mfma_chunk(fo, vq[dc], ad);
          }
          s[mt] = as;
          dp[mt] = ad;
        }
        const long key = kb + 16 * wv + c16;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const f32x4 l2 = *reinterpret_cast<const f32x4 *>(s_lse2 + mt * 16 + 4 * g);
          const f32x4 dd = *reinterpret_cast<const f32x4 *>(s_dd + mt * 16 + 4 * g);
          const int4 ps = *reinterpret_cast<const int4 *>(s_pos + mt * 16 + 4 * g);
          const int pv[4] = {ps.x, ps.y, ps.z, ps.w};
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const float pr = key <= pv[ii] ? __builtin_amdgcn_exp2f(fmaf(s[mt][ii], cs, -l2[ii])) : 0.f;
            s[mt][ii] = pr;
            dp[mt][ii] = pr * (dp[mt][ii] - dd[ii]) * dscale;
          }
        }
        // dV_w += P^T dO, dK_w += dS^T Q over the tile's 32 row-heads
        {
          const F ap = acc_frag(s[0], s[1], tagp);
          const F as = acc_frag(dp[0], dp[1], tagp);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            if constexpr (L::ES == 2) {
              dv[dt] = mfma_chunk(ap, tr_frag_rm<L>(s_do, dt * 16, g, lane), dv[dt]);
              dk[dt] = mfma_chunk(as, tr_frag_rm<L>(s_q, dt * 16, g, lane), dk[dt]);
            } else {
              const int d = dt * 16 + c16;
              dv[dt] = mfma_chunk(ap, tr_frag(s_dot + d * L::TROW, g), dv[dt]);
              dk[dt] = mfma_chunk(as, tr_frag(s_qt + d * L::TROW, g), dk[dt]);
            }
          }
        }
        // dS (as the matrix cores take it) to LDS for the dq product
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
            put1(s_ds + (mt * 16 + 4 * g + ii) * L::SROW + (16 * wv + c16) * L::ES, dp[mt][ii], tagp);
        __syncthreads();

        // dq for this wave's DSL columns over the whole block
        unsigned char *so = s_o[wv];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          F fa[KS];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            fa[ks] = load_frag(reinterpret_cast<const E *>(s_ds + (mt * 16 + c16) * L::SROW + (ks * 32 + g * 8) * L::ES));
#pragma unroll
          for (int nt = 0; nt < QN; ++nt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = mfma_chunk(fa[ks], ktf[nt][ks], acc);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
              put1(so + (mt * 16 + 4 * g + ii) * L::OROW + (nt * 16 + c16) * L::ES, acc[ii], tagp);
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // wave-private buffer: in-order LDS
        {
          // A fixed number of stores per lane with no branch, so that the compiler counts
          // them: the next tile's wait for its Q / dO loads (issued before these stores)
          // then leaves the stores in flight instead of waiting for all memory operations.
          // Row-heads past the chunk's entries store the tile's first row of the same head
          // again (the same bytes to the same address).
          constexpr int PPR = DSL * L::ES / 16;  // 16-byte pieces per row-head
          constexpr int NST = TR * PPR / 64;
          static_assert(TR * PPR % 64 == 0, "dq pieces must fill whole waves");
          u32x4 val[NST];
          u32x4 *dst[NST];
          // 80-byte rows of 4 pieces: each 16-lane group of the 16-byte reads takes four
          // rows whose bank groups do not overlap (rows 4 j + group for j = 0..3).
          constexpr bool REMAP = L::ES == 2 && PPR == 4 && L::OROW == 80;
          int qrow = lane >> 2;
          if constexpr (REMAP) {
            const int hi = qrow >> 3, lo = qrow & 7, inner = ((lo + 2) >> 2) & 1;
            const int grp = 2 * hi + inner, j = inner ? lo - 2 : (lo < 2 ? lo : lo - 4);
            qrow = 4 * j + grp;
          }
#pragma unroll
          for (int i = 0; i < NST; ++i) {
            const int pc = lane + 64 * i, off = pc % PPR;
            int m = REMAP ? 16 * i + qrow : pc / PPR;
            if (tt * RPT + (m >> log2g) >= n_e) m &= G - 1;
            const int en = s_list[tt * RPT + (m >> log2g)];
            const long pss = ((((long)b * a.h_kv + r) * a.n_q + (en >> 6)) * a.top_k + (en & 63)) * G + (m & (G - 1));
            val[i] = *reinterpret_cast<const u32x4 *>(so + m * L::OROW + off * 16);
            dst[i] = reinterpret_cast<u32x4 *>(reinterpret_cast<unsigned char *>(a.part_o) +
                                               (pss * DH + wv * DSL) * L::ES + off * 16);
          }
#pragma unroll
          for (int i = 0; i < NST; ++i) __builtin_nontemporal_store(val[i], dst[i]);
        }
        if (tt + 1 < n_tiles) {  // uniform
          // This tile's reads of the staging buffers ended at the barrier before the dq
          // product, which reads only dS and registers.
          write_tile();
          load_tile(min(tt + 2, n_tiles - 1));  // in flight over the next tile (no branch)
          __syncthreads();
        }
      }
    }
    if (cur >= 0) flush();
  }
}

// ---------------------------------------------------------------- dq merge

// Slots whose loads a dq_merge thread issues together: all 32 of a row for bf16 (6.49
// against 6.67 ms with 8 at 128K; 150 VGPRs, three waves per SIMD), 8 for fp32, whose
// 32-slot batch would take every register.
template <typename E> constexpr int DQ_BATCH = sizeof(E) == 2 ? 32 : 8;

// Each (b, r, row) is summed by LPR = G * DH / 8 consecutive threads, 8 outputs of one head
// each, over the row's valid slots in slot order.
template <typename E, int DH, int U>
__global__ __launch_bounds__(256) void dq_merge(KvArgs a, BwdArgs w, int log2g) {
  const int G = 1 << log2g;
  const int lpr_log2 = log2g + (DH == 128 ? 4 : 3);
  const int span = min(1 << lpr_log2, 64);
  const long gl = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = gl >> lpr_log2;
  const long rows = (long)a.batch * a.h_kv * a.n_q;
  const int lane = threadIdx.x & 63;
  const int j = (int)(gl & ((1L << lpr_log2) - 1));

  uint64_t mask = 0;
  for (int m = 0; m * span < a.top_k; ++m) {
    const int sl = m * span + (lane & (span - 1));
    const int c = (sl < a.top_k && row < rows) ? a.sel[row * a.top_k + sl] : -1;
    const uint64_t bl = ballot(c >= 0 && c < a.n_blocks);
    const uint64_t bits = span == 64 ? bl : ((bl >> (lane & ~(span - 1))) & ((1ull << span) - 1));
    mask |= bits << (m * span);
  }
  if (row >= rows) return;

  const int hd = j / (DH / 8), d0 = (j % (DH / 8)) * 8;
  const E *pbase = reinterpret_cast<const E *>(a.part_o) + (row * a.top_k * G + hd) * DH + d0;
  float acc[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) acc[x] = 0.f;
  // U slots' loads in flight together, added in slot order (the same bits as one at a time)
  uint64_t v = mask;
  while (v) {
    int sl[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      sl[u] = v ? __builtin_ctzll(v) : -1;
      v &= v - 1;  // no-op once v is 0
    }
    // Every load is issued (a slot past the row's last reads slot 0 again and is masked
    // below): loads under branches would go one at a time.
    if constexpr (sizeof(E) == 2) {
      u32x4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        x[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(pbase + (long)max(sl[u], 0) * G * DH));
#pragma unroll
      for (int u = 0; u < U; ++u) pin(x[u]);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = sl[u] >= 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = acc[2 * e] + __uint_as_float(x[u][e] << 16);
          const float hi = acc[2 * e + 1] + __uint_as_float(x[u][e] & 0xffff0000u);
          acc[2 * e] = ok ? lo : acc[2 * e];
          acc[2 * e + 1] = ok ? hi : acc[2 * e + 1];
        }
      }
    } else {
      f32x4 lo[U], hi[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(pbase + (long)max(sl[u], 0) * G * DH);
        lo[u] = __builtin_nontemporal_load(p);
        hi[u] = __builtin_nontemporal_load(p + 1);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        pin(lo[u]);
        pin(hi[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = sl[u] >= 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a0 = acc[e] + lo[u][e], a1 = acc[4 + e] + hi[u][e];
          acc[e] = ok ? a0 : acc[e];
          acc[4 + e] = ok ? a1 : acc[4 + e];
        }
      }
    }
  }
  const int t = (int)(row % a.n_q);
  const long br = row / a.n_q;
  const int r = (int)(br % a.h_kv), b = (int)(br / a.h_kv);
  E *o = reinterpret_cast<E *>(w.dq) + (((long)b * a.h_q + r * G + hd) * a.n_q + t) * DH + d0;
  if constexpr (sizeof(E) == 2) {
    *reinterpret_cast<u32x4 *>(o) = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                          pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
  } else {
    float *of = reinterpret_cast<float *>(o);
    *reinterpret_cast<f32x4 *>(of) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4 *>(of + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
}

// ---------------------------------------------------------------- dk, dv reduce

// One workgroup per (b, r, block): sums the block's segment partials over its lists (one
// per row segment) in chunk order and writes the block's valid key rows of dk and dv.
template <typename E, int DH, int BS>
__global__ __launch_bounds__(256) void dkv_reduce(KvArgs a, BwdArgs w) {
  constexpr int PIECES = 2 * BS * DH / 4;  // float4 pieces: dK, then dV
  constexpr int PT = PIECES / 256;
  const int c = (int)(blockIdx.x % a.n_blocks);
  const long br = blockIdx.x / a.n_blocks;
  const int r = (int)(br % a.h_kv), b = (int)(br / a.h_kv);
  f32x4 acc[PT];
#pragma unroll
  for (int u = 0; u < PT; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int sg = 0; sg < a.n_seg; ++sg) {
    const long i = bwd_list_index(a, b, r, sg, c);
    const int x0 = a.coff[i], x1 = a.coff[i + 1];
    for (int x = x0; x < x1; x = (x / w.run + 1) * w.run) {  // one segment per run it meets
      const long slot = x % w.run == 0 ? x / w.run : w.run_slots + i;
      const f32x4 *src = reinterpret_cast<const f32x4 *>(w.dkv + slot * (2L * BS * DH));
#pragma unroll
      for (int u = 0; u < PT; ++u) {
        const f32x4 y = __builtin_nontemporal_load(src + threadIdx.x + 256 * u);
        acc[u] += y;
      }
    }
  }
  const long plane = ((long)b * a.h_kv + r) * (long)a.cap * DH;
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int pc = threadIdx.x + 256 * u;
    const int which = pc / (BS * DH / 4), rem = pc % (BS * DH / 4);
    const int key = rem / (DH / 4), d0 = (rem % (DH / 4)) * 4;
    const long j = (long)c * BS + key;
    if (j < a.n_k) {
      E *dst = reinterpret_cast<E *>(which ? w.dv : w.dk) + plane + j * DH + d0;
      if constexpr (sizeof(E) == 2)
        *reinterpret_cast<u32x2 *>(dst) = u32x2{pack_bf16x2(acc[u][0], acc[u][1]), pack_bf16x2(acc[u][2], acc[u][3])};
      else
        *reinterpret_cast<f32x4 *>(dst) = acc[u];
    }
  }
}

template <typename E, int DH, int BS>
hipError_t run_bwd(const KvArgs &a, const BwdArgs &w, const void *o, int log2g, long max_runs,
                   int stages, hipStream_t s) {
  if (stages & BWD_STAGE_ROWDOT) {
    const long hrows = (long)a.batch * a.h_q * a.n_q;
    hipLaunchKernelGGL((bwd_rowdot<E, DH>), dim3((unsigned)((hrows * (DH / 8) + 255) / 256)), dim3(256),
                       0, s, reinterpret_cast<const E *>(o), reinterpret_cast<const E *>(w.dout),
                       const_cast<float *>(w.dsum), hrows);
  }
  if (!(stages & (BWD_STAGE_BLOCKS | BWD_STAGE_MERGE))) return hipGetLastError();
  static const int per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kv_bwd<E, DH, BS>, BwdLds<E, DH, BS>::NT, 0) !=
            hipSuccess || n < 1)
      n = 1;
    return n;
  }();
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  // one round of the workgroups that fit on the device at once; runs are claimed
  const unsigned grid = (unsigned)std::max(1L, std::min(max_runs, (long)per_cu * cus));
  if (stages & BWD_STAGE_BLOCKS) {
    KvArgs b = a;
    b.claim = a.cnt + 2L * a.n_seg * a.batch * a.h_kv * a.n_blocks;  // zeroed by the plan
    hipLaunchKernelGGL((kv_bwd<E, DH, BS>), dim3(grid), dim3(BwdLds<E, DH, BS>::NT), 0, s, b, w, log2g);
  }
  if (!(stages & BWD_STAGE_MERGE)) return hipGetLastError();
  const long threads = (long)a.batch * a.h_kv * a.n_q * ((long)DH << log2g) / 8;
  hipLaunchKernelGGL((dq_merge<E, DH, DQ_BATCH<E>>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a, w,
                     log2g);
  hipLaunchKernelGGL((dkv_reduce<E, DH, BS>), dim3((unsigned)((long)a.batch * a.h_kv * a.n_blocks)),
                     dim3(256), 0, s, a, w);
  return hipGetLastError();
}

}  // namespace

constexpr int BWD_RUN = 8;  // chunks per kv_bwd work item

size_t kv_bwd_workspace_bytes(long batch, long h_kv, long n_q, long top_k, long n_blocks, long group,
                              long d_h, long block_size, long elem_bytes, BwdLayout *lay) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  BwdLayout L;
  size_t o = kv_workspace_bytes(batch, h_kv, n_q, top_k, n_blocks, group, d_h, elem_bytes, &L.kv);
  const long seg_rows = kv_segment_rows(batch, h_kv, n_q, top_k, n_blocks, group, d_h, elem_bytes);
  const long n_seg = (n_q + seg_rows - 1) / seg_rows;
  const long NB = n_seg * batch * h_kv * n_blocks;
  const long slots = batch * h_kv * n_q * top_k;
  const long max_chunks = (slots + CHUNK - 1) / CHUNK + NB;
  L.run = BWD_RUN;
  L.max_runs = (max_chunks + BWD_RUN - 1) / BWD_RUN;
  L.dsum = o;  o += al((size_t)(batch * h_kv * group * n_q) * 4);
  L.dkv = o;   o += al((size_t)(L.max_runs + NB) * (size_t)(2 * block_size * d_h) * 4);
  L.total = o;
  if (lay) *lay = L;
  return o;
}

hipError_t launch_attn_backward(const KvArgs &a, const BwdLayout &lay, unsigned char *ws, const void *o,
                                const void *dout, const float *lse, void *dq, void *dk, void *dv,
                                int dtype, int d_h, int stages, hipStream_t s) {
  int lg = 0;
  while ((1 << lg) < a.h_q / a.h_kv) ++lg;
  BwdArgs w{dout, lse, reinterpret_cast<const float *>(ws + lay.dsum), reinterpret_cast<float *>(ws + lay.dkv),
            dq, dk, dv, (float)(1.0 / std::sqrt((double)d_h)), lay.run, lay.max_runs};
#define MSA_BWD(E, DH)                                                                  \
  if (a.block_size == 32) return run_bwd<E, DH, 32>(a, w, o, lg, lay.max_runs, stages, s); \
  return run_bwd<E, DH, 64>(a, w, o, lg, lay.max_runs, stages, s);
  if (dtype == 0) {
    if (d_h == 64) { MSA_BWD(float, 64) }
    MSA_BWD(float, 128)
  }
  if (d_h == 64) { MSA_BWD(bf16_t, 64) }
  MSA_BWD(bf16_t, 128)
#undef MSA_BWD
}

}  // namespace msa
