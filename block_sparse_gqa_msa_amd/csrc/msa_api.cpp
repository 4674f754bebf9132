// msa_api.cpp -- the C ABI declared in include/msa.h: argument validation, workspace
// sizing and kernel launches. Every check runs on the host before anything is enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "msa.h"
#include "msa_internal.hpp"

namespace {

thread_local std::string g_error;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int ok() {
  g_error.clear();
  return MSA_OK;
}

bool pow2_upto(int x, int hi) { return x >= 1 && x <= hi && (x & (x - 1)) == 0; }

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

long long n_blocks(const msa_shape &s) { return ((long long)s.n_k + s.block_size - 1) / s.block_size; }
long long n_runs(const msa_shape &s) { return (n_blocks(s) + msa::RUN_BLOCKS - 1) / msa::RUN_BLOCKS; }
int cap_of(const msa_shape &s) { return s.kv_capacity ? s.kv_capacity : s.n_k; }

// Checks shared by every entry point.
int check_shape(const msa_shape *s) {
  if (!s) return fail(MSA_ERR_INVALID_ARG, "shape is NULL");
  if (s->batch < 0 || s->n_q < 0 || s->n_k < 0 || s->q_start < 0)
    return fail(MSA_ERR_INVALID_ARG, "batch, n_q, n_k and q_start must be >= 0 (got %d, %d, %d, %d)",
                s->batch, s->n_q, s->n_k, s->q_start);
  if ((long long)s->q_start + s->n_q > s->n_k)
    return fail(MSA_ERR_INVALID_ARG, "q_start + n_q (%lld) exceeds n_k (%d)",
                (long long)s->q_start + s->n_q, s->n_k);
  if (s->kv_capacity != 0 && s->kv_capacity < s->n_k)
    return fail(MSA_ERR_INVALID_ARG, "kv_capacity (%d) is neither 0 nor >= n_k (%d)", s->kv_capacity, s->n_k);
  if (s->h_kv < 1 || s->h_q < 1 || s->h_q % s->h_kv)
    return fail(MSA_ERR_INVALID_ARG, "h_q (%d) must be a positive multiple of h_kv (%d)", s->h_q, s->h_kv);
  if (s->top_k < 1) return fail(MSA_ERR_INVALID_ARG, "top_k must be >= 1 (got %d)", s->top_k);
  if (s->block_size < 1) return fail(MSA_ERR_INVALID_ARG, "block_size must be >= 1");
  if (s->dtype != MSA_F32 && s->dtype != MSA_BF16)
    return fail(MSA_ERR_UNSUPPORTED, "dtype %d is not MSA_F32 or MSA_BF16", s->dtype);
  if (s->block_size != 32 && s->block_size != 64)
    return fail(MSA_ERR_UNSUPPORTED, "block_size %d not in {32, 64}", s->block_size);
  if (s->top_k > 64) return fail(MSA_ERR_UNSUPPORTED, "top_k %d > 64", s->top_k);
  if (!pow2_upto(s->h_kv, 16)) return fail(MSA_ERR_UNSUPPORTED, "h_kv %d not in {1,2,4,8,16}", s->h_kv);
  if (!pow2_upto(s->h_q / s->h_kv, 16))
    return fail(MSA_ERR_UNSUPPORTED, "h_q / h_kv = %d not in {1,2,4,8,16}", s->h_q / s->h_kv);
  return MSA_OK;
}

// No rows to compute (batch or n_q is 0): every call is a no-op that succeeds.
bool empty(const msa_shape &s) { return s.batch == 0 || s.n_q == 0; }

int topk_chunks(const msa_shape &s) {
  if (s.top_k == 1) return 1;  // the local block alone: no ranking
  // candidate blocks of the last row: its local block index
  const long long last_local = ((long long)s.q_start + s.n_q - 1) / s.block_size;
  const long long n = last_local < 1 ? 1 : (last_local + msa::TOPK_CHUNK - 1) / msa::TOPK_CHUNK;
  return (int)n;
}

struct IndexWs {
  // bytes of: the block maxima, each of the two candidate arrays, the run keys, the index
  // kernel's spare destination; laid out in that order
  size_t bmax, cand, rkey, spare, total;
  size_t dec_cand;  // fused decode path: candidate pairs of every index-select workgroup
  bool fused;       // the fused decode path applies
};

// Fused decode selection: one query row, its candidates fit one merge pass.
int decode_select_wgs(const msa_shape &s) {
  const long long blocks = (long long)s.q_start / s.block_size + 1;
  return (int)((blocks + msa::SEL_NBLK - 1) / msa::SEL_NBLK);
}
bool fused_decode_ok(const msa_shape &s) {
  return s.n_q == 1 && s.top_k > 1 &&
         (long long)decode_select_wgs(s) * (s.top_k - 1) <= msa::TOPK_CHUNK;
}

int index_ws(const msa_shape &s, bool with_bmax, bool with_runs, IndexWs *w) {
  const long long rows = (long long)s.batch * s.h_kv * s.n_q;
  const int nch = topk_chunks(s);
  if (nch > 1 && (long long)nch * (s.top_k - 1) > msa::TOPK_CHUNK)
    return fail(MSA_ERR_UNSUPPORTED, "too many candidate blocks (%lld) for top_k %d",
                ((long long)s.q_start + s.n_q - 1) / s.block_size, s.top_k);
  w->bmax = with_bmax ? align_up((size_t)rows * (size_t)n_blocks(s) * sizeof(float)) : 0;
  w->cand = nch > 1 ? align_up((size_t)rows * nch * (s.top_k - 1) * 4) : 0;
  // run keys: prefill rows with more than one chunk of candidates (index kernel to top-k)
  w->rkey = with_runs && nch > 1 && s.n_q > 1
                ? align_up(((size_t)rows * (size_t)n_runs(s) + 1) * sizeof(uint32_t))
                : 0;
  w->spare = with_runs && s.n_q > 1 ? 256 : 0;
  w->total = w->bmax + 2 * w->cand + w->rkey + w->spare;
  w->fused = fused_decode_ok(s);
  w->dec_cand = w->fused ? align_up((size_t)rows * decode_select_wgs(s) * (s.top_k - 1) * 4) : 0;
  if (2 * w->dec_cand > w->total) w->total = 2 * w->dec_cand;
  return MSA_OK;
}

int check_index_dims(const msa_shape &s) {
  if (s.d_idx != 32 && s.d_idx != 64) return fail(MSA_ERR_UNSUPPORTED, "d_idx %d not in {32, 64}", s.d_idx);
  return MSA_OK;
}

int check_attn_dims(const msa_shape &s) {
  if (s.d_h != 64 && s.d_h != 128) return fail(MSA_ERR_UNSUPPORTED, "d_h %d not in {64, 128}", s.d_h);
  return MSA_OK;
}

int decode_splits(const msa_shape &s) { return s.top_k; }  // one selected block per split

bool is_decode(const msa_shape &s) { return s.n_q == 1 && s.q_start == s.n_k - 1; }

size_t attn_prefill_ws(const msa_shape &s, msa::KvLayout *lay) {
  return msa::kv_workspace_bytes(s.batch, s.h_kv, s.n_q, s.top_k, n_blocks(s), s.h_q / s.h_kv,
                                 s.d_h, s.dtype == MSA_F32 ? 4 : 2, lay);
}

int kv_seg_rows(const msa_shape &s) {
  return msa::kv_segment_rows(s.batch, s.h_kv, s.n_q, s.top_k, n_blocks(s), s.h_q / s.h_kv, s.d_h,
                              s.dtype == MSA_F32 ? 4 : 2);
}

int check_prefill_limits(const msa_shape &s) {
  const long long entries = (long long)s.batch * s.h_kv * s.n_q * s.top_k;
  const long long n_seg = (s.n_q + kv_seg_rows(s) - 1) / kv_seg_rows(s);
  const long long merge_threads = (long long)s.batch * s.h_q * s.n_q * (s.d_h / 8);
  if (entries >= (1LL << 31) || s.n_q >= (1 << 25) || merge_threads >= (1LL << 32) ||
      n_seg * s.batch * s.h_kv * n_blocks(s) >= (1LL << 30))
    return fail(MSA_ERR_UNSUPPORTED, "prefill too large for one call (%lld selection entries); "
                "split the query rows over several calls", entries);
  return MSA_OK;
}

size_t attn_decode_ws(const msa_shape &s) {
  const size_t parts = (size_t)s.batch * s.h_q * decode_splits(s);
  return align_up(parts * s.d_h * sizeof(float)) + align_up(parts * 2 * sizeof(float));
}

// msa_decode_step's workspace: arrival counters, then the index branch's workspace, then
// the attention's (decode partials).
struct StepWs {
  size_t cnt, idx, attn, total;
};
int step_ws(const msa_shape &s, StepWs *w) {
  IndexWs iw;
  int rc = index_ws(s, true, true, &iw);
  if (rc) return rc;
  w->cnt = align_up((size_t)s.batch * s.h_kv * sizeof(int32_t));
  w->idx = align_up(iw.total);
  w->attn = attn_decode_ws(s);
  w->total = w->cnt + w->idx + w->attn;
  return MSA_OK;
}

// Workgroups per (sequence, group) in the fused decode kernel: enough that every wave
// attends about one selected block, no more than about one workgroup per compute unit.
int finish_subs(const msa_shape &s) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const long long pairs = (long long)s.batch * s.h_kv;
  const long long by_blocks = (s.top_k + 3) / 4;
  const long long by_cus = cus / pairs;
  long long subs = by_blocks < by_cus ? by_blocks : by_cus;
  if (subs > msa::FINISH_MAX_SUBS) subs = msa::FINISH_MAX_SUBS;
  return subs < 1 ? 1 : (int)subs;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int key_chunk_prefill(const msa_shape &s) {
  const long long tq = 256 / s.h_kv;
  const long long tiles = ((long long)s.n_q + tq - 1) / tq * s.batch;
  const long long avg_keys = (long long)s.q_start + s.n_q / 2 + 1;
  int kc = 8192;
  while (kc > 512 && tiles * ((avg_keys + kc - 1) / kc) < 4096) kc /= 2;
  const long long keys = (long long)s.q_start + s.n_q;
  while ((keys + kc - 1) / kc > 65535) kc *= 2;  // key chunks are the grid's y dimension
  return kc;
}

int key_chunk_decode(const msa_shape &s) {
  const long long keys = (long long)s.q_start + 1;
  int kc = 4096;
  while (kc > 256 && s.batch * ((keys + kc - 1) / kc) < 2048) kc /= 2;
  return kc;
}

// The allocation-free decode step's workspace: one array per GPU, held until the process
// ends. Host code never uses this name as an address (on the host it is only a stand-in);
// device_scratch() takes each GPU's address once, with that GPU current.
static __device__ __align__(256) unsigned char scratch[MSA_DECODE_STEP_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

int device_scratch(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MSA_ERR_UNSUPPORTED, "device ordinal %d beyond %d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e, "address of the decode-step scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}

}  // namespace

extern "C" {

int msa_abi_version(void) { return 1; }

const char *msa_last_error(void) { return g_error.c_str(); }

int msa_index_topk_workspace_size(const msa_shape *shape, size_t *bytes) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_index_dims(*shape))) return rc;
  if (!bytes) return fail(MSA_ERR_INVALID_ARG, "bytes is NULL");
  if (empty(*shape)) {
    *bytes = 0;
    return ok();
  }
  IndexWs w;
  if ((rc = index_ws(*shape, true, true, &w))) return rc;
  *bytes = w.total;
  return ok();
}

// Shared by msa_index_topk, its two stages and the two split calls. With rkey (prefill only),
// the index kernel also writes run keys; its key chunks are then whole runs.
static int launch_scores(const msa_shape &s, const void *q_idx, const void *k_idx, float *bmax,
                         uint32_t *rkey, float *spare, hipStream_t st) {
  msa::IndexArgs ia{q_idx, k_idx, bmax, s.batch, s.n_q, s.n_k, s.q_start, s.h_kv,
                    (int)n_blocks(s), cap_of(s), 0, nullptr, nullptr, s.top_k};
  ia.spare = spare;
  hipError_t e;
  if (s.n_q == 1) {
    ia.key_chunk = key_chunk_decode(s);
    e = msa::launch_index_decode(ia, s.dtype, s.d_idx, s.block_size, st);
  } else {
    ia.key_chunk = key_chunk_prefill(s);
    if (rkey) {  // both powers of two: the larger is a whole number of runs
      ia.rkey = rkey;
      ia.n_runs = (int)n_runs(s);
      ia.key_chunk = std::max(ia.key_chunk, msa::RUN_BLOCKS * s.block_size);
    }
    e = msa::launch_index_prefill(ia, s.dtype, s.d_idx, s.block_size, st);
  }
  return e == hipSuccess ? MSA_OK : hip_fail(e, "index kernel launch");
}

static int launch_select(const msa_shape &s, const float *bmax, int32_t *sel, unsigned char *cand,
                         size_t cand_bytes, const uint32_t *rkey, hipStream_t st) {
  msa::TopkArgs ta{bmax, sel, reinterpret_cast<uint32_t *>(cand),
                   reinterpret_cast<int32_t *>(cand + cand_bytes), s.batch, s.n_q, s.q_start,
                   s.h_kv, (int)n_blocks(s), s.block_size, s.top_k, topk_chunks(s),
                   msa::TOPK_CHUNK, 0};
  ta.rkey = rkey;
  ta.n_runs = rkey ? (int)n_runs(s) : 0;
  hipError_t e = msa::launch_topk(ta, st);
  return e == hipSuccess ? MSA_OK : hip_fail(e, "top-k kernel launch");
}

enum { INDEX_STAGE_SCORES = 1, INDEX_STAGE_SELECT = 2, INDEX_STAGE_ALL = 3 };

// msa_index_topk and its two stages: the same workspace layout and kernels either way.
static int index_topk(const msa_shape *shape, const void *q_idx, const void *k_idx, int32_t *sel,
                      float *block_scores, void *workspace, size_t workspace_bytes, void *stream,
                      int stages) {
  int rc = check_shape(shape);
  if (rc) return rc;
  const msa_shape &s = *shape;
  if ((rc = check_index_dims(s))) return rc;
  if (empty(s)) return ok();
  if ((stages & INDEX_STAGE_SCORES) && (!q_idx || !k_idx))
    return fail(MSA_ERR_INVALID_ARG, "q_idx and k_idx must be non-NULL");
  if ((stages & INDEX_STAGE_SELECT) && !sel) return fail(MSA_ERR_INVALID_ARG, "sel must be non-NULL");
  IndexWs w;
  if ((rc = index_ws(s, block_scores == nullptr, true, &w))) return rc;
  if (w.total && (!workspace || workspace_bytes < w.total))
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", w.total,
                workspace ? workspace_bytes : (size_t)0);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  unsigned char *ws = reinterpret_cast<unsigned char *>(workspace);
  if (!block_scores && w.fused) {  // decode: first selection stage inside the index kernel
    uint32_t *ck = reinterpret_cast<uint32_t *>(ws);
    int32_t *ci = reinterpret_cast<int32_t *>(ws + w.dec_cand);
    if (stages & INDEX_STAGE_SCORES) {
      msa::IndexArgs ia{q_idx, k_idx, nullptr, s.batch, s.n_q, s.n_k, s.q_start, s.h_kv,
                        (int)n_blocks(s), cap_of(s), 0, ck, ci, s.top_k};
      hipError_t e = msa::launch_index_select_decode(ia, s.dtype, s.d_idx, s.block_size, st);
      if (e != hipSuccess) return hip_fail(e, "index-select kernel launch");
    }
    if (stages & INDEX_STAGE_SELECT) {
      msa::TopkArgs ta{nullptr, sel, ck, ci, s.batch, s.n_q, s.q_start, s.h_kv, (int)n_blocks(s),
                       s.block_size, s.top_k, decode_select_wgs(s), msa::SEL_NBLK, 1};
      hipError_t e = msa::launch_topk_final(ta, st);
      if (e != hipSuccess) return hip_fail(e, "top-k merge launch");
    }
    return ok();
  }
  float *bmax = block_scores ? block_scores : reinterpret_cast<float *>(ws);
  uint32_t *rkey = w.rkey ? reinterpret_cast<uint32_t *>(ws + w.bmax + 2 * w.cand) : nullptr;
  float *spare = w.spare ? reinterpret_cast<float *>(ws + w.bmax + 2 * w.cand + w.rkey) : nullptr;
  if (stages & INDEX_STAGE_SCORES) {
    if (block_scores) {
      const long long rows = (long long)s.batch * s.h_kv * s.n_q;
      hipError_t e = msa::launch_fill(block_scores, (size_t)rows * (size_t)n_blocks(s), -INFINITY, st);
      if (e != hipSuccess) return hip_fail(e, "block score fill");
    }
    if ((rc = launch_scores(s, q_idx, k_idx, bmax, rkey, spare, st))) return rc;
  }
  if (stages & INDEX_STAGE_SELECT) {
    if ((rc = launch_select(s, bmax, sel, ws + w.bmax, w.cand, rkey, st))) return rc;
  }
  return ok();
}

int msa_index_topk(const msa_shape *shape, const void *q_idx, const void *k_idx, int32_t *sel,
                   float *block_scores, void *workspace, size_t workspace_bytes, void *stream) {
  return index_topk(shape, q_idx, k_idx, sel, block_scores, workspace, workspace_bytes, stream,
                    INDEX_STAGE_ALL);
}

int msa_index_topk_scores(const msa_shape *shape, const void *q_idx, const void *k_idx,
                          float *block_scores, void *workspace, size_t workspace_bytes,
                          void *stream) {
  return index_topk(shape, q_idx, k_idx, nullptr, block_scores, workspace, workspace_bytes,
                    stream, INDEX_STAGE_SCORES);
}

int msa_index_topk_select(const msa_shape *shape, const float *block_scores, int32_t *sel,
                          void *workspace, size_t workspace_bytes, void *stream) {
  // The select stage only reads block_scores (when given): the stage-1 call wrote them.
  return index_topk(shape, nullptr, nullptr, sel, const_cast<float *>(block_scores), workspace,
                    workspace_bytes, stream, INDEX_STAGE_SELECT);
}

int msa_index_block_scores(const msa_shape *shape, const void *q_idx, const void *k_idx,
                           float *block_scores, void *stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  const msa_shape &s = *shape;
  if ((rc = check_index_dims(s))) return rc;
  if (empty(s)) return ok();
  if (!q_idx || !k_idx || !block_scores)
    return fail(MSA_ERR_INVALID_ARG, "q_idx, k_idx and block_scores must be non-NULL");
  if ((rc = launch_scores(s, q_idx, k_idx, block_scores, nullptr, nullptr,
                          reinterpret_cast<hipStream_t>(stream))))
    return rc;
  return ok();
}

int msa_topk_workspace_size(const msa_shape *shape, size_t *bytes) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!bytes) return fail(MSA_ERR_INVALID_ARG, "bytes is NULL");
  if (empty(*shape)) {
    *bytes = 0;
    return ok();
  }
  IndexWs w;
  if ((rc = index_ws(*shape, false, false, &w))) return rc;
  *bytes = w.total;
  return ok();
}

int msa_topk_from_block_scores(const msa_shape *shape, const float *block_scores, int32_t *sel,
                               void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  const msa_shape &s = *shape;
  if (empty(s)) return ok();
  if (!block_scores || !sel) return fail(MSA_ERR_INVALID_ARG, "block_scores and sel must be non-NULL");
  IndexWs w;
  if ((rc = index_ws(s, false, false, &w))) return rc;
  if (w.total && (!workspace || workspace_bytes < w.total))
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", w.total,
                workspace ? workspace_bytes : (size_t)0);
  if ((rc = launch_select(s, block_scores, sel, reinterpret_cast<unsigned char *>(workspace),
                          w.cand, nullptr, reinterpret_cast<hipStream_t>(stream))))
    return rc;
  return ok();
}

int msa_sparse_attn_workspace_size(const msa_shape *shape, size_t *bytes) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_attn_dims(*shape))) return rc;
  if (!bytes) return fail(MSA_ERR_INVALID_ARG, "bytes is NULL");
  if (empty(*shape)) {
    *bytes = 0;
    return ok();
  }
  if ((rc = check_prefill_limits(*shape))) return rc;
  *bytes = attn_prefill_ws(*shape, nullptr);
  if (is_decode(*shape)) {  // either entry point may be called for a decode shape
    const size_t d = attn_decode_ws(*shape);
    if (d > *bytes) *bytes = d;
  }
  return ok();
}

// An attention call with no rows: the dimensions must still be supported; nothing runs.
static int empty_attn_call(const msa_shape &s) {
  const int rc = check_attn_dims(s);
  return rc ? rc : ok();
}

// Validates a prefill-attention call and fills the kernel arguments over the caller's
// workspace; the pointers a stage does not use may be NULL.
static int prefill_args(const msa_shape *shape, void *workspace, size_t workspace_bytes,
                        msa::KvArgs *out) {
  int rc = check_shape(shape);
  if (rc) return rc;
  const msa_shape &s = *shape;
  if ((rc = check_attn_dims(s))) return rc;
  if ((rc = check_prefill_limits(s))) return rc;
  msa::KvLayout lay;
  const size_t need = attn_prefill_ws(s, &lay);
  if (!workspace || workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  unsigned char *ws = reinterpret_cast<unsigned char *>(workspace);
  const int seg_rows = kv_seg_rows(s);
  const int n_seg = (s.n_q + seg_rows - 1) / seg_rows;
  const long long NB = (long long)n_seg * s.batch * s.h_kv * n_blocks(s);
  int32_t *cnt = reinterpret_cast<int32_t *>(ws + lay.cnt);
  *out = msa::KvArgs{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, cnt, cnt + NB,
                     reinterpret_cast<int32_t *>(ws + lay.boff), reinterpret_cast<int32_t *>(ws + lay.coff),
                     reinterpret_cast<int32_t *>(ws + lay.list), reinterpret_cast<int32_t *>(ws + lay.cmap),
                     reinterpret_cast<long *>(ws + lay.tile_sum), ws + lay.part_o,
                     reinterpret_cast<float *>(ws + lay.part_ml), s.batch, s.n_q, s.n_k, s.q_start,
                     s.h_q, s.h_kv, s.block_size, s.top_k, cap_of(s), (int)n_blocks(s), seg_rows,
                     n_seg, (float)(1.4426950408889634 / std::sqrt((double)s.d_h))};
  return MSA_OK;
}

static int run_prefill(const msa_shape &s, const msa::KvArgs &a, int stages, void *stream) {
  hipError_t e = msa::launch_attn_prefill_kv(a, s.dtype, s.d_h, stages,
                                             reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "prefill attention launch");
  return ok();
}

int msa_sparse_attn_prefill(const msa_shape *shape, const void *q, const void *k, const void *v,
                            const int32_t *sel, void *o, float *lse, void *workspace,
                            size_t workspace_bytes, void *stream) {
  msa::KvArgs a;
  int rc = check_shape(shape);
  if (rc) return rc;
  if (empty(*shape)) return empty_attn_call(*shape);
  if (!q || !k || !v || !sel || !o) return fail(MSA_ERR_INVALID_ARG, "q, k, v, sel and o must be non-NULL");
  if ((rc = prefill_args(shape, workspace, workspace_bytes, &a))) return rc;
  a.q = q; a.k = k; a.v = v; a.sel = sel; a.o = o; a.lse = lse;
  return run_prefill(*shape, a, msa::KV_STAGE_ALL, stream);
}

int msa_sparse_attn_prefill_plan(const msa_shape *shape, const int32_t *sel, void *workspace,
                                 size_t workspace_bytes, void *stream) {
  msa::KvArgs a;
  int rc = check_shape(shape);
  if (rc) return rc;
  if (empty(*shape)) return empty_attn_call(*shape);
  if (!sel) return fail(MSA_ERR_INVALID_ARG, "sel must be non-NULL");
  if ((rc = prefill_args(shape, workspace, workspace_bytes, &a))) return rc;
  a.sel = sel;
  return run_prefill(*shape, a, msa::KV_STAGE_PLAN, stream);
}

int msa_sparse_attn_prefill_partials(const msa_shape *shape, const void *q, const void *k,
                                     const void *v, void *workspace, size_t workspace_bytes,
                                     void *stream) {
  msa::KvArgs a;
  int rc = check_shape(shape);
  if (rc) return rc;
  if (empty(*shape)) return empty_attn_call(*shape);
  if (!q || !k || !v) return fail(MSA_ERR_INVALID_ARG, "q, k and v must be non-NULL");
  if ((rc = prefill_args(shape, workspace, workspace_bytes, &a))) return rc;
  a.q = q; a.k = k; a.v = v;
  return run_prefill(*shape, a, msa::KV_STAGE_ATTEND, stream);
}

int msa_sparse_attn_prefill_merge(const msa_shape *shape, const int32_t *sel, void *o, float *lse,
                                  void *workspace, size_t workspace_bytes, void *stream) {
  msa::KvArgs a;
  int rc = check_shape(shape);
  if (rc) return rc;
  if (empty(*shape)) return empty_attn_call(*shape);
  if (!sel || !o) return fail(MSA_ERR_INVALID_ARG, "sel and o must be non-NULL");
  if ((rc = prefill_args(shape, workspace, workspace_bytes, &a))) return rc;
  a.sel = sel; a.o = o; a.lse = lse;
  return run_prefill(*shape, a, msa::KV_STAGE_MERGE, stream);
}

int msa_index_kl(const msa_shape *shape, const void *q, const void *k, const void *q_idx,
                 const void *k_idx, const int32_t *sel, const float *lse, float *kl,
                 float *lse_idx, void *workspace, size_t workspace_bytes, void *stream) {
  msa::KvArgs a;
  int rc = check_shape(shape);
  if (rc) return rc;
  const msa_shape &s = *shape;
  if ((rc = check_index_dims(s))) return rc;
  if (empty(s)) return empty_attn_call(s);
  if (!q || !k || !q_idx || !k_idx || !sel || !lse || !kl)
    return fail(MSA_ERR_INVALID_ARG, "q, k, q_idx, k_idx, sel, lse and kl must be non-NULL");
  if ((rc = prefill_args(shape, workspace, workspace_bytes, &a))) return rc;
  a.q = q; a.k = k; a.sel = sel;
  if ((rc = run_prefill(s, a, msa::KV_STAGE_PLAN, stream))) return rc;
  msa::KvLayout lay;
  attn_prefill_ws(s, &lay);
  unsigned char *ws = reinterpret_cast<unsigned char *>(workspace);
  const msa::KlArgs kk{q_idx, k_idx, lse, kl, lse_idx, reinterpret_cast<float4 *>(ws + lay.part_o),
                       reinterpret_cast<float2 *>(ws + lay.part_ml),
                       (float)(1.0 / std::sqrt((double)s.d_idx))};
  hipError_t e = msa::launch_index_kl(a, kk, s.dtype, s.d_h, s.d_idx,
                                      reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "alignment loss launch");
  return ok();
}

static size_t attn_backward_ws(const msa_shape &s, msa::BwdLayout *lay) {
  return msa::kv_bwd_workspace_bytes(s.batch, s.h_kv, s.n_q, s.top_k, n_blocks(s), s.h_q / s.h_kv,
                                     s.d_h, s.block_size, s.dtype == MSA_F32 ? 4 : 2, lay);
}

int msa_sparse_attn_backward_workspace_size(const msa_shape *shape, size_t *bytes) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_attn_dims(*shape))) return rc;
  if (!bytes) return fail(MSA_ERR_INVALID_ARG, "bytes is NULL");
  if (empty(*shape)) {
    *bytes = 0;
    return ok();
  }
  if ((rc = check_prefill_limits(*shape))) return rc;
  *bytes = attn_backward_ws(*shape, nullptr);
  return ok();
}

// Validates a backward call and fills the kernel arguments over the caller's workspace
// (the lists live at its start, laid out as for the prefill).
static int backward_args(const msa_shape *shape, void *workspace, size_t workspace_bytes,
                         msa::KvArgs *a, msa::BwdLayout *lay) {
  int rc = check_shape(shape);
  if (rc) return rc;
  const msa_shape &s = *shape;
  if ((rc = check_attn_dims(s))) return rc;
  if ((rc = check_prefill_limits(s))) return rc;
  const size_t need = attn_backward_ws(s, lay);
  if (!workspace || workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  return prefill_args(shape, workspace, workspace_bytes, a);
}

static int run_backward(const msa_shape &s, const msa::KvArgs &a, const msa::BwdLayout &lay,
                        void *workspace, const void *o, const void *dout, const float *lse,
                        void *dq, void *dk, void *dv, int stages, void *stream) {
  hipError_t e = msa::launch_attn_backward(a, lay, reinterpret_cast<unsigned char *>(workspace), o,
                                           dout, lse, dq, dk, dv, s.dtype, s.d_h, stages,
                                           reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attention backward launch");
  return ok();
}

int msa_sparse_attn_backward(const msa_shape *shape, const void *q, const void *k, const void *v,
                             const int32_t *sel, const void *o, const float *lse, const void *dout,
                             void *dq, void *dk, void *dv, void *workspace, size_t workspace_bytes,
                             void *stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  const msa_shape &s = *shape;
  if (empty(s)) return empty_attn_call(s);
  if (!q || !k || !v || !sel || !o || !lse || !dout || !dq || !dk || !dv)
    return fail(MSA_ERR_INVALID_ARG, "q, k, v, sel, o, lse, dout, dq, dk and dv must be non-NULL");
  msa::KvArgs a;
  msa::BwdLayout lay;
  if ((rc = backward_args(shape, workspace, workspace_bytes, &a, &lay))) return rc;
  a.q = q; a.k = k; a.v = v; a.sel = sel;
  if ((rc = run_prefill(s, a, msa::KV_STAGE_PLAN, stream))) return rc;
  return run_backward(s, a, lay, workspace, o, dout, lse, dq, dk, dv, msa::BWD_STAGE_ALL, stream);
}

int msa_sparse_attn_backward_plan(const msa_shape *shape, const int32_t *sel, const void *o,
                                  const void *dout, void *workspace, size_t workspace_bytes,
                                  void *stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  const msa_shape &s = *shape;
  if (empty(s)) return empty_attn_call(s);
  if (!sel || !o || !dout) return fail(MSA_ERR_INVALID_ARG, "sel, o and dout must be non-NULL");
  msa::KvArgs a;
  msa::BwdLayout lay;
  if ((rc = backward_args(shape, workspace, workspace_bytes, &a, &lay))) return rc;
  a.sel = sel;
  if ((rc = run_prefill(s, a, msa::KV_STAGE_PLAN, stream))) return rc;
  return run_backward(s, a, lay, workspace, o, dout, nullptr, nullptr, nullptr, nullptr,
                      msa::BWD_STAGE_ROWDOT, stream);
}

int msa_sparse_attn_backward_partials(const msa_shape *shape, const void *q, const void *k,
                                      const void *v, const float *lse, const void *dout,
                                      void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  const msa_shape &s = *shape;
  if (empty(s)) return empty_attn_call(s);
  if (!q || !k || !v || !lse || !dout)
    return fail(MSA_ERR_INVALID_ARG, "q, k, v, lse and dout must be non-NULL");
  msa::KvArgs a;
  msa::BwdLayout lay;
  if ((rc = backward_args(shape, workspace, workspace_bytes, &a, &lay))) return rc;
  a.q = q; a.k = k; a.v = v;
  return run_backward(s, a, lay, workspace, nullptr, dout, lse, nullptr, nullptr, nullptr,
                      msa::BWD_STAGE_BLOCKS, stream);
}

int msa_sparse_attn_backward_merge(const msa_shape *shape, const int32_t *sel, void *dq, void *dk,
                                   void *dv, void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  const msa_shape &s = *shape;
  if (empty(s)) return empty_attn_call(s);
  if (!sel || !dq || !dk || !dv) return fail(MSA_ERR_INVALID_ARG, "sel, dq, dk and dv must be non-NULL");
  msa::KvArgs a;
  msa::BwdLayout lay;
  if ((rc = backward_args(shape, workspace, workspace_bytes, &a, &lay))) return rc;
  a.sel = sel;
  return run_backward(s, a, lay, workspace, nullptr, nullptr, nullptr, dq, dk, dv,
                      msa::BWD_STAGE_MERGE, stream);
}

int msa_index_project(const msa_shape *shape, int32_t d_model, const void *x, const void *w_qidx,
                      const void *w_kidx, void *q_idx, void *k_idx, void *stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  const msa_shape &s = *shape;
  if ((rc = check_index_dims(s))) return rc;
  if (d_model < 64 || d_model % 64)
    return fail(MSA_ERR_UNSUPPORTED, "d_model %d is not a positive multiple of 64", d_model);
  if (empty(s)) return ok();
  if (!x || !w_qidx || !w_kidx || !q_idx || !k_idx)
    return fail(MSA_ERR_INVALID_ARG, "x, w_qidx, w_kidx, q_idx and k_idx must be non-NULL");
  if ((long long)s.batch * s.n_q >= (1LL << 36))
    return fail(MSA_ERR_UNSUPPORTED, "too many rows (%lld) for one call",
                (long long)s.batch * s.n_q);
  const msa::ProjArgs a{x, w_qidx, w_kidx, q_idx, k_idx, s.batch, s.n_q, s.q_start, s.h_kv,
                        d_model, cap_of(s), (s.h_kv + 1) * s.d_idx};
  hipError_t e = msa::launch_index_project(a, s.dtype, s.d_idx, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "index projection launch");
  return ok();
}

int msa_sparse_attn_decode(const msa_shape *shape, const void *q, const void *k_cache,
                           const void *v_cache, const int32_t *sel, void *o, float *lse,
                           void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  const msa_shape &s = *shape;
  if ((rc = check_attn_dims(s))) return rc;
  if (s.n_q != 1 || s.q_start != s.n_k - 1)
    return fail(MSA_ERR_INVALID_ARG, "decode needs n_q == 1 and q_start == n_k - 1 (got %d, %d, n_k %d)",
                s.n_q, s.q_start, s.n_k);
  if (empty(s)) return ok();
  if (!q || !k_cache || !v_cache || !sel || !o)
    return fail(MSA_ERR_INVALID_ARG, "q, k_cache, v_cache, sel and o must be non-NULL");
  const size_t need = attn_decode_ws(s);
  if (!workspace || workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  const int S = decode_splits(s);
  const size_t parts = (size_t)s.batch * s.h_q * S;
  unsigned char *ws = reinterpret_cast<unsigned char *>(workspace);
  msa::AttnArgs a{q, k_cache, v_cache, sel, o, lse,
                  reinterpret_cast<float *>(ws),
                  reinterpret_cast<float *>(ws + align_up(parts * s.d_h * sizeof(float))),
                  s.batch, 1, s.n_k, s.q_start, s.h_q, s.h_kv, s.block_size, s.top_k, cap_of(s),
                  S, (s.top_k + S - 1) / S,
                  (float)(1.4426950408889634 / std::sqrt((double)s.d_h))};
  hipError_t e = msa::launch_attn_decode(a, s.dtype, s.d_h, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode attention launch");
  return ok();
}

int msa_decode_step_workspace_size(const msa_shape *shape, size_t *bytes) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_index_dims(*shape)) || (rc = check_attn_dims(*shape))) return rc;
  if (!bytes) return fail(MSA_ERR_INVALID_ARG, "bytes is NULL");
  if (empty(*shape)) {
    *bytes = 0;
    return ok();
  }
  StepWs w;
  if ((rc = step_ws(*shape, &w))) return rc;
  *bytes = w.total;
  return ok();
}

// Validation shared by the decode-step entry points (nothing is enqueued on failure).
static int check_decode_step(const msa_shape *shape, const void *q, const void *k_cache,
                             const void *v_cache, const void *q_idx, const void *k_idx,
                             const int32_t *sel, const void *o) {
  int rc = check_shape(shape);
  if (rc) return rc;
  const msa_shape &s = *shape;
  if ((rc = check_index_dims(s)) || (rc = check_attn_dims(s))) return rc;
  if (s.n_q != 1 || s.q_start != s.n_k - 1)
    return fail(MSA_ERR_INVALID_ARG, "decode needs n_q == 1 and q_start == n_k - 1 (got %d, %d, n_k %d)",
                s.n_q, s.q_start, s.n_k);
  if (empty(s)) return MSA_OK;
  if (!q || !k_cache || !v_cache || !q_idx || !k_idx || !sel || !o)
    return fail(MSA_ERR_INVALID_ARG, "q, k_cache, v_cache, q_idx, k_idx, sel and o must be non-NULL");
  return MSA_OK;
}

int msa_decode_step(const msa_shape *shape, const void *q, const void *k_cache, const void *v_cache,
                    const void *q_idx, const void *k_idx, int32_t *sel, void *o, float *lse,
                    void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_decode_step(shape, q, k_cache, v_cache, q_idx, k_idx, sel, o);
  if (rc) return rc;
  const msa_shape &s = *shape;
  if (empty(s)) return ok();
  StepWs w;
  if ((rc = step_ws(s, &w))) return rc;
  if (!workspace || workspace_bytes < w.total)
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", w.total,
                workspace ? workspace_bytes : (size_t)0);
  unsigned char *ws = reinterpret_cast<unsigned char *>(workspace);
  unsigned char *ws_idx = ws + w.cnt, *ws_attn = ws + w.cnt + w.idx;
  if (!fused_decode_ok(s)) {  // k == 1, or too many candidates for one merge: the two calls
    if ((rc = msa_index_topk(shape, q_idx, k_idx, sel, nullptr, ws_idx, w.idx, stream))) return rc;
    return msa_sparse_attn_decode(shape, q, k_cache, v_cache, sel, o, lse, ws_attn, w.attn, stream);
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  IndexWs iw;
  if ((rc = index_ws(s, true, true, &iw))) return rc;
  uint32_t *ck = reinterpret_cast<uint32_t *>(ws_idx);
  int32_t *ci = reinterpret_cast<int32_t *>(ws_idx + iw.dec_cand);
  int32_t *cnt = reinterpret_cast<int32_t *>(ws);
  msa::IndexArgs ia{q_idx, k_idx, nullptr, s.batch, s.n_q, s.n_k, s.q_start, s.h_kv,
                    (int)n_blocks(s), cap_of(s), 0, ck, ci, s.top_k};
  ia.zero = cnt;
  ia.n_zero = s.batch * s.h_kv;
  hipError_t e = msa::launch_index_select_decode(ia, s.dtype, s.d_idx, s.block_size, st);
  if (e != hipSuccess) return hip_fail(e, "index-select kernel launch");
  const int subs = finish_subs(s);
  const int S = decode_splits(s);
  const size_t parts = (size_t)s.batch * s.h_q * S;  // >= pairs * subs * G: subs <= top_k
  msa::AttnArgs a{q, k_cache, v_cache, sel, o, lse,
                  reinterpret_cast<float *>(ws_attn),
                  reinterpret_cast<float *>(ws_attn + align_up(parts * s.d_h * sizeof(float))),
                  s.batch, 1, s.n_k, s.q_start, s.h_q, s.h_kv, s.block_size, s.top_k, cap_of(s),
                  S, (s.top_k + S - 1) / S,
                  (float)(1.4426950408889634 / std::sqrt((double)s.d_h))};
  msa::FinishArgs f{ck, ci, sel, cnt, decode_select_wgs(s), subs};
  e = msa::launch_decode_finish(a, f, s.dtype, s.d_h, st);
  if (e != hipSuccess) return hip_fail(e, "decode finish launch");
  return ok();
}

int msa_decode_step_noalloc(const msa_shape *shape, const void *q, const void *k_cache,
                            const void *v_cache, const void *q_idx, const void *k_idx, int32_t *sel,
                            void *o, float *lse, void *stream) {
  int rc = check_decode_step(shape, q, k_cache, v_cache, q_idx, k_idx, sel, o);
  if (rc) return rc;
  if (empty(*shape)) return ok();
  StepWs w;
  if ((rc = step_ws(*shape, &w))) return rc;
  if (w.total > MSA_DECODE_STEP_SCRATCH_BYTES)
    return fail(MSA_ERR_WORKSPACE, "this decode step needs %zu bytes of workspace, more than the "
                "%zu-byte scratch array of msa_decode_step_noalloc; use msa_decode_step",
                w.total, (size_t)MSA_DECODE_STEP_SCRATCH_BYTES);
  void *scratch_ptr = nullptr;
  if ((rc = device_scratch(&scratch_ptr))) return rc;
  return msa_decode_step(shape, q, k_cache, v_cache, q_idx, k_idx, sel, o, lse, scratch_ptr,
                         MSA_DECODE_STEP_SCRATCH_BYTES, stream);
}

}  // extern "C"
