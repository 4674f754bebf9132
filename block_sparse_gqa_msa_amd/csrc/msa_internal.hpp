// msa_internal.hpp -- launchers shared between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

struct IndexArgs {
  const void *q_idx;  // [B, R, n_q, DI]
  const void *k_idx;  // [B, cap, DI]
  float *bmax;        // [B, R, n_q, n_blocks]
  int batch, n_q, n_k, q_start, h_kv, n_blocks, cap;
  int key_chunk;      // keys per workgroup (multiple of 64)
  // decode selection fused into the index kernel (index_select_decode only):
  uint32_t *cand_key;  // [B, R, n_wg, top_k - 1] best blocks of each workgroup's range
  int32_t *cand_idx;
  int top_k;
  int32_t *zero = nullptr;  // index_select_decode: n_zero words cleared for the next kernel
  int n_zero = 0;
  // index_pool_prefill, when set: per (b, group, row) and aligned run of RUN_BLOCKS blocks,
  // the run key: order_key of the run's largest block maximum. One more word after the
  // array takes the stores of columns past the rows.
  uint32_t *rkey = nullptr;  // [B, R, n_q, n_runs] + 1
  int n_runs = 0;
  // index_pool_prefill: 16 bytes (16-byte aligned) that take the stores of columns past
  // the rows, or null; with it the maxima are flushed with a fixed number of stores.
  float *spare = nullptr;
};

constexpr int SEL_NBLK = 256;  // key blocks per fused decode index-select workgroup

struct TopkArgs {
  const float *bmax;   // [B, R, n_q, n_blocks]
  int32_t *sel;        // [B, R, n_q, k]
  uint32_t *cand_key;  // [problems, n_chunks, k-1]  (two-level path only)
  int32_t *cand_idx;   // [problems, n_chunks, k-1]
  int batch, n_q, q_start, h_kv, n_blocks, block_size, top_k;
  int n_chunks;        // candidate chunks per problem (stride of cand_key / cand_idx)
  int chunk_blocks;    // blocks per chunk (TOPK_CHUNK, or SEL_NBLK after the fused decode kernel)
  int final_all;       // merge pass also writes problems with a single chunk (fused decode path)
  // Run keys from the index kernel (see IndexArgs::rkey), or null. With them, problems with
  // more than TOPK_CHUNK candidates read only the runs that can hold a winner.
  const uint32_t *rkey = nullptr;  // [B, R, n_q, n_runs]
  int n_runs = 0;
};

struct AttnArgs {
  const void *q;       // [B, H, n_q, DH]
  const void *k;       // [B, R, cap, DH]
  const void *v;       // [B, R, cap, DH]
  const int32_t *sel;  // [B, R, n_q, top_k]
  void *o;             // [B, H, n_q, DH]
  float *lse;          // [B, H, n_q] or null
  float *part_o;       // decode partials [B, H, S, DH]
  float *part_ml;      // decode partials [B, H, S, 2] (max in log2 units, sum)
  int batch, n_q, n_k, q_start, h_q, h_kv, block_size, top_k, cap;
  int splits;          // decode: number of splits S
  int blocks_per_split;
  float scale_log2;    // log2(e) / sqrt(DH)
};

constexpr int FINISH_MAX_SUBS = 16;  // workgroups per (sequence, group) in decode_finish

struct FinishArgs {          // decode: final selection, attention and merge in one kernel
  const uint32_t *cand_key;  // [B, R, n_wg, top_k - 1] per-range winners of index_select_decode
  const int32_t *cand_idx;
  int32_t *sel;              // [B, R, top_k] out
  int32_t *cnt;              // [B, R] arrival counters, zero when the kernel starts
  int n_wg;                  // key ranges per sequence (the candidates' stride)
  int subs;                  // workgroups per (sequence, group)
};

struct KvArgs {          // KV-outer prefill attention
  const void *q, *k, *v;
  const int32_t *sel;
  void *o;
  float *lse;
  int32_t *cnt;          // [NB] entries per (b, r, block); cursor follows it: [NB]
  int32_t *cursor;
  int32_t *boff;         // [NB + 1] first entry of each block's list
  int32_t *coff;         // [NB + 1] first chunk of each block
  int32_t *list;         // [entries] row * 64 + slot, grouped by block
  int32_t *cmap;         // [chunks] list index of each chunk
  long *tile_sum;        // [2 * scan tiles] scan scratch
  void *part_o;          // [B*R*n_q*top_k][G][DH] unnormalised partial outputs (dtype)
  float *part_ml;        // [B*R*n_q*top_k][G][2] (max in log2 units, sum)
  int batch, n_q, n_k, q_start, h_q, h_kv, block_size, top_k, cap, n_blocks;
  int seg_rows;          // lists are keyed (r, row segment, b, block), group-major
  int n_seg;
  float scale_log2;
  int32_t *claim = nullptr;  // next-chunk counter of the persistent kernels: zeroed by the
                             // plan (it follows cnt and cursor), reset by the last claim
};

constexpr int KV_CHUNK = 256;  // list entries per work item of the KV-outer kernels

// The alignment loss over the KV-outer lists (the KvArgs of the same shape carry q, k, sel,
// the lists and the sizes).
struct KlArgs {
  const void *q_idx;  // [B, R, n_q, DI]
  const void *k_idx;  // [B, cap, DI]
  const float *lse;   // [B, H, n_q] main-branch log-sum-exp (natural log) from the forward
  float *kl;          // [B, R, n_q] out
  float *lse_idx;     // [B, R, n_q] out, or null
  float4 *part;       // [B*R*n_q*top_k] per selection: (sum t ln t, sum t S^idx, sum t, 0)
  float2 *part_ml;    // [B*R*n_q*top_k] per selection: index scores' (max, sum), log2 units
  float scale_idx;    // 1 / sqrt(d_idx)
};

struct KvLayout {
  size_t cnt, boff, coff, cmap, tile_sum, list, part_o, part_ml, total;
};

// Rows per list segment for a prefill of this size (a multiple of the list-build tile).
int kv_segment_rows(long batch, long h_kv, long n_q, long top_k, long n_blocks, long group,
                    long d_h, long elem_bytes);
size_t kv_workspace_bytes(long batch, long h_kv, long n_q, long top_k, long n_blocks, long group,
                          long d_h, long elem_bytes, KvLayout *lay);

// The index branch's projections from hidden states x [B, n_q, d_model].
struct ProjArgs {
  const void *x;    // [B, n_q, d_model]
  const void *w_q;  // [h_kv * d_idx, d_model], one row per output
  const void *w_k;  // [d_idx, d_model]
  void *q_idx;      // [B, h_kv, n_q, d_idx] out
  void *k_idx;      // [B, cap, d_idx]: rows q_start .. q_start + n_q - 1 written
  int batch, n_q, q_start, h_kv, d_model, cap;
  int n_cols;       // (h_kv + 1) * d_idx
};

// Backward workspace: the prefill lists (KvLayout; part_o holds the dq partials), D per
// (b, h, t), and one fp32 dK/dV partial per (run, list) segment of the backward kernel.
struct BwdLayout {
  KvLayout kv;
  size_t dsum, dkv, total;
  int run;        // chunks per run
  long max_runs;  // runs at most (segment slots [0, max_runs) start runs; list i's own is max_runs + i)
};
size_t kv_bwd_workspace_bytes(long batch, long h_kv, long n_q, long top_k, long n_blocks, long group,
                              long d_h, long block_size, long elem_bytes, BwdLayout *lay);

constexpr int TOPK_CHUNK = 2048;  // candidate blocks one wave ranks at a time
constexpr int RUN_BLOCKS = 32;    // blocks per run key (aligned runs: blocks 32 r .. 32 r + 31)

// Each launcher validates nothing (the C-ABI layer did) and returns the launch status.
hipError_t launch_fill(float *p, size_t n, float value, hipStream_t s);
hipError_t launch_index_prefill(const IndexArgs &a, int dtype, int d_idx, int block_size,
                                hipStream_t s);
hipError_t launch_index_decode(const IndexArgs &a, int dtype, int d_idx, int block_size,
                               hipStream_t s);
hipError_t launch_topk(const TopkArgs &a, hipStream_t s);
hipError_t launch_topk_final(const TopkArgs &a, hipStream_t s);
hipError_t launch_index_select_decode(const IndexArgs &a, int dtype, int d_idx, int block_size,
                                      hipStream_t s);
// Stages of the prefill attention: list build from sel, per-selection partials, merge.
enum { KV_STAGE_PLAN = 1, KV_STAGE_ATTEND = 2, KV_STAGE_MERGE = 4, KV_STAGE_ALL = 7 };
hipError_t launch_attn_prefill_kv(const KvArgs &a, int dtype, int d_h, int stages, hipStream_t s);
hipError_t launch_attn_decode(const AttnArgs &a, int dtype, int d_h, hipStream_t s);
hipError_t launch_decode_finish(const AttnArgs &a, const FinishArgs &f, int dtype, int d_h,
                                hipStream_t s);
// Alignment loss from the lists a plan stage built: per-selection sums, then the merge.
hipError_t launch_index_kl(const KvArgs &a, const KlArgs &k, int dtype, int d_h, int d_idx,
                           hipStream_t s);

hipError_t launch_index_project(const ProjArgs &a, int dtype, int d_idx, hipStream_t s);
// Main-branch gradients for a fixed selection, after the list build (plan stage): D per
// (b, h, t), the per-block gradients, then the dq merge and the dk/dv reduction.
enum { BWD_STAGE_ROWDOT = 1, BWD_STAGE_BLOCKS = 2, BWD_STAGE_MERGE = 4, BWD_STAGE_ALL = 7 };
hipError_t launch_attn_backward(const KvArgs &a, const BwdLayout &lay, unsigned char *ws, const void *o,
                                const void *dout, const float *lse, void *dq, void *dk, void *dv,
                                int dtype, int d_h, int stages, hipStream_t s);

}  // namespace msa
