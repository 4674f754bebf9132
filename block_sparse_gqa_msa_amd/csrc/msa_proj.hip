// msa_proj.hip -- the index branch's two projections from the hidden states.
//
// "MiniMax-M3: MSA 技术报告速读", section 核心机制 (索引分支): the index branch adds two
// projection matrices to GQA, an index query with one head per group and an index key
// shared by the groups. For hidden states x [B, n, d_model] and weights stored one row per
// output ([h_kv * d_idx, d_model] and [d_idx, d_model]):
//   q_idx[b, r, t, :] = x[b, t] . w_q[r * d_idx + d]   (written [B, h_kv, n, d_idx])
//   k_idx[b, q_start + t, :] = x[b, t] . w_k[d]       (appended to the cache rows of the
//                                                       call's positions)
// One product over the concatenated output columns (h_kv + 1) * d_idx: a workgroup takes
// 128 rows of x (64 for fp32) and all the output columns up to 320, a quarter per wave;
// x is staged in LDS 64 columns of d_model at a time, and each wave reads its weight
// fragments straight from memory (the weights are a few MB and stay in L2). Every
// workgroup reads the whole weight once per row range, so more rows per workgroup means
// less L2 traffic.
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {
namespace {

constexpr int PJ_K = 64;  // d_model columns per staged tile

// MT 16-row tiles per workgroup (all four waves share them) and NT 16-column output tiles
// per wave: a workgroup covers 16 * MT rows and 64 * NT output columns.
template <typename E, int DI, int MT, int NT>
__global__ __launch_bounds__(256) void index_project(ProjArgs a) {
  using F = typename Frag<E>::type;
  constexpr int ES = (int)sizeof(E);
  constexpr int PM = 16 * MT;                   // rows per workgroup
  // x rows in LDS: a fragment read's 16 lanes of one LDS pass take rows 0-7 at 16-byte
  // piece p and rows 8-15 at piece p + 1; bf16 rows of 128 bytes stay unpadded with the
  // piece XORed by row & 7, which puts the 16 on distinct bank groups (16 bytes of padding
  // left two on one); fp32 rows keep the padding.
  constexpr bool XSW = ES == 2 && PJ_K * ES == 128;
  constexpr int XROW = XSW ? PJ_K * ES : PJ_K * ES + 16;
  constexpr int PPR = PJ_K * ES / 16;           // 16-byte pieces per staged row
  constexpr int PT = PM * PPR / 256;            // pieces per thread
  __shared__ __attribute__((aligned(16))) unsigned char s_x[2][PM * XROW];
  auto x_at = [](int row, int piece) { return row * XROW + (XSW ? piece ^ (row & 7) : piece) * 16; };

  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const long rows = (long)a.batch * a.n_q;
  const long row0 = (long)blockIdx.x * PM;
  const int col0 = (blockIdx.y * 4 + wv) * 16 * NT;
  const bool active = col0 < a.n_cols;  // uniform over the wave
  const int qcols = a.h_kv * DI;
  const E *x = reinterpret_cast<const E *>(a.x);
  const E *wrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int c = min(col0 + nt * 16 + c16, a.n_cols - 1);
    wrow[nt] = c < qcols ? reinterpret_cast<const E *>(a.w_q) + (long)c * a.d_model
                         : reinterpret_cast<const E *>(a.w_k) + (long)(c - qcols) * a.d_model;
  }

  u32x4 xp[PT];
  auto load_x = [&](int k0) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int pc = tid + 256 * i;
      const long gr = min(row0 + pc / PPR, rows - 1);  // rows past the end repeat the last
      xp[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
          reinterpret_cast<const unsigned char *>(x + gr * a.d_model + k0) + (pc % PPR) * 16));
    }
  };
  // this wave's weight fragments of one staged tile; loaded right after the previous
  // tile's last use so they arrive over the barrier and the staging
  F wf[2][NT];
  auto load_w = [&](int k0) {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) wf[kc][nt] = load_frag(wrow[nt] + k0 + kc * 32 + g * 8);
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // x tiles are double-buffered in LDS: tile s + 1 is written while tile s is read, and the
  // loads of tile s + 2 have a whole tile's products to arrive in.
  auto store_x = [&](unsigned char *dst) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int pc = tid + 256 * i;
      *reinterpret_cast<u32x4 *>(dst + x_at(pc / PPR, pc % PPR)) = xp[i];
    }
  };
  const int n_tiles = a.d_model / PJ_K;
  load_x(0);
  load_w(0);
  store_x(s_x[0]);
  load_x(n_tiles > 1 ? PJ_K : 0);
  __syncthreads();
  for (int tile = 0; tile < n_tiles; ++tile) {
    const unsigned char *cur = s_x[tile & 1];
    if (active) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const F af = load_frag(reinterpret_cast<const E *>(cur + x_at(mt * 16 + c16, (kc * 32 + g * 8) * ES / 16)));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma_chunk(af, wf[kc][nt], acc[mt][nt]);
        }
    }
    // unconditional loads: past the last tile they re-read the last one
    const int k1 = min(tile + 1, n_tiles - 1) * PJ_K, k2 = min(tile + 2, n_tiles - 1) * PJ_K;
    load_w(k1);
    store_x(s_x[(tile + 1) & 1]);  // tile + 1 (its buffer was last read before the barrier)
    load_x(k2);
    __syncthreads();
  }
  // Outputs go through LDS one 16-row tile at a time (a wave-private slice of the x
  // buffers, free after the last barrier), then out as 16-byte pieces of 8 (bf16) or 4
  // (fp32) consecutive columns: a piece never straddles a group's d_idx columns or the
  // query / key boundary.
  constexpr int OROW = 16 * NT * ES + 16;
  static_assert(4 * 16 * OROW <= 2 * PM * XROW, "output staging fits the x buffers");
  unsigned char *so = s_x[0] + wv * 16 * OROW;
  constexpr int PE = 16 / ES, PPO = 16 * NT / PE;  // elements per piece, pieces per row
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (active) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          unsigned char *dst = so + (4 * g + i) * OROW + (nt * 16 + c16) * ES;
          if constexpr (ES == 2)
            *reinterpret_cast<uint16_t *>(dst) = (uint16_t)(pack_bf16x2(acc[mt][nt][i], 0.f) & 0xffffu);
          else
            *reinterpret_cast<float *>(dst) = acc[mt][nt][i];
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // wave-private: in-order LDS
      for (int pc = lane; pc < 16 * PPO; pc += 64) {
        const int rr = pc / PPO, c = col0 + (pc % PPO) * PE;
        const long gr = row0 + mt * 16 + rr;
        if (c >= a.n_cols || gr >= rows) continue;
        const long b = gr / a.n_q, t = gr % a.n_q;
        const long off = c < qcols ? (((b * a.h_kv + c / DI) * a.n_q + t) * DI + c % DI)
                                   : ((b * a.cap + a.q_start + t) * DI + (c - qcols));
        E *dst = reinterpret_cast<E *>(c < qcols ? a.q_idx : a.k_idx) + off;
        *reinterpret_cast<u32x4 *>(dst) = *reinterpret_cast<const u32x4 *>(so + rr * OROW + (pc % PPO) * 16);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next tile's writes
    }
  }
}

template <typename E, int DI, int MT, int NT>
void launch_pj(const ProjArgs &a, hipStream_t s) {
  const long rows = (long)a.batch * a.n_q;
  const dim3 grid((unsigned)((rows + 16 * MT - 1) / (16 * MT)),
                  (unsigned)((a.n_cols + 64 * NT - 1) / (64 * NT)));
  hipLaunchKernelGGL((index_project<E, DI, MT, NT>), grid, dim3(256), 0, s, a);
}

// Column tiles per wave: the output columns spread over the four waves, at most five
// 16-column tiles each (wider outputs take several workgroups per row range).
template <typename E, int DI, int MT>
void launch_pj_cols(const ProjArgs &a, hipStream_t s) {
  const int per_wave = (a.n_cols + 63) / 64;
  switch (per_wave < 5 ? per_wave : 5) {
    case 1: launch_pj<E, DI, MT, 1>(a, s); break;
    case 2: launch_pj<E, DI, MT, 2>(a, s); break;
    case 3: launch_pj<E, DI, MT, 3>(a, s); break;
    case 4: launch_pj<E, DI, MT, 4>(a, s); break;
    default: launch_pj<E, DI, MT, 5>(a, s); break;
  }
}

}  // namespace

hipError_t launch_index_project(const ProjArgs &a, int dtype, int d_idx, hipStream_t s) {
  if (dtype == 0) {  // fp32 fragments are twice the registers: half the rows per workgroup
    if (d_idx == 32)
      launch_pj_cols<float, 32, 4>(a, s);
    else
      launch_pj_cols<float, 64, 4>(a, s);
  } else {
    if (d_idx == 32)
      launch_pj_cols<bf16_t, 32, 8>(a, s);
    else
      launch_pj_cols<bf16_t, 64, 8>(a, s);
  }
  return hipGetLastError();
}

}  // namespace msa
