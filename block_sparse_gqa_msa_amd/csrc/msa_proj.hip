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
// 64 rows of x and up to four 64-column output tiles (one per wave); x is staged in LDS 64
// columns of d_model at a time, and each wave reads its weight fragments straight from
// memory (the weights are a few MB and stay in L2), one stage ahead.
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {
namespace {

constexpr int PJ_M = 64;  // rows per workgroup
constexpr int PJ_K = 64;  // d_model columns per staged tile
constexpr int PJ_N = 64;  // output columns per wave

template <typename E, int DI>
__global__ __launch_bounds__(256) void index_project(ProjArgs a) {
  using F = typename Frag<E>::type;
  constexpr int ES = (int)sizeof(E);
  constexpr int XROW = PJ_K * ES + 16;
  constexpr int PPR = PJ_K * ES / 16;           // 16-byte pieces per staged row
  constexpr int PT = PJ_M * PPR / 256;          // pieces per thread
  __shared__ __attribute__((aligned(16))) unsigned char s_x[PJ_M * XROW];

  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const long rows = (long)a.batch * a.n_q;
  const long row0 = (long)blockIdx.x * PJ_M;
  const int col0 = (blockIdx.y * 4 + wv) * PJ_N;
  const bool active = col0 < a.n_cols;  // uniform over the wave
  const int qcols = a.h_kv * DI;
  const E *x = reinterpret_cast<const E *>(a.x);
  const E *wrow[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
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
  F wf[2][4], wn[2][4];
  auto load_w = [&](int k0, F (&dst)[2][4]) {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) dst[kc][nt] = load_frag(wrow[nt] + k0 + kc * 32 + g * 8);
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_x(0);
  load_w(0, wf);
  for (int k0 = 0; k0 < a.d_model; k0 += PJ_K) {
    __syncthreads();  // the previous tile's reads are done
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int pc = tid + 256 * i;
      *reinterpret_cast<u32x4 *>(s_x + (pc / PPR) * XROW + (pc % PPR) * 16) = xp[i];
    }
    __syncthreads();
    // the next tile's loads stay in flight over this one (the last tile reloads itself)
    const int kn = k0 + PJ_K < a.d_model ? k0 + PJ_K : k0;
    load_x(kn);
    load_w(kn, wn);
    if (active) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        F af[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          af[mt] = load_frag(reinterpret_cast<const E *>(s_x + (mt * 16 + c16) * XROW + (kc * 32 + g * 8) * ES));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_chunk(af[mt], wf[kc][nt], acc[mt][nt]);
      }
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) wf[kc][nt] = wn[kc][nt];
  }
  if (!active) return;

  // lane (c16, g) holds output column 16 nt + c16 of rows 16 mt + 4 g + i
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int c = col0 + nt * 16 + c16;
    if (c >= a.n_cols) continue;
    const bool is_q = c < qcols;
    const int r = c / DI, d = c % DI, dk = c - qcols;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const long gr = row0 + mt * 16 + 4 * g + i;
        if (gr >= rows) continue;
        const long b = gr / a.n_q, t = gr % a.n_q;
        const long off = is_q ? (((b * a.h_kv + r) * a.n_q + t) * DI + d)
                              : ((b * a.cap + a.q_start + t) * DI + dk);
        E *dst = reinterpret_cast<E *>(is_q ? a.q_idx : a.k_idx) + off;
        if constexpr (ES == 2)
          *reinterpret_cast<uint16_t *>(dst) = (uint16_t)(pack_bf16x2(acc[mt][nt][i], 0.f) & 0xffffu);
        else
          *reinterpret_cast<float *>(dst) = acc[mt][nt][i];
      }
  }
}

}  // namespace

hipError_t launch_index_project(const ProjArgs &a, int dtype, int d_idx, hipStream_t s) {
  const long rows = (long)a.batch * a.n_q;
  const dim3 grid((unsigned)((rows + PJ_M - 1) / PJ_M), (unsigned)((a.n_cols + 4 * PJ_N - 1) / (4 * PJ_N)));
  if (dtype == 0) {
    if (d_idx == 32)
      hipLaunchKernelGGL((index_project<float, 32>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((index_project<float, 64>), grid, dim3(256), 0, s, a);
  } else {
    if (d_idx == 32)
      hipLaunchKernelGGL((index_project<bf16_t, 32>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((index_project<bf16_t, 64>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace msa
