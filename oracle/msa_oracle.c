/*
 * msa_oracle.c -- plain, slow, fp64 CPU oracle for MiniMax Sparse Attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark load this file's library. The GPU library never links,
 * includes or calls it, and it shares no code, header or table with the GPU
 * path.
 *
 * What it computes, step by step, follows the page "MiniMax-M3: MSA 技术报告速读"
 * (mloasisblog.com/blog/ML/minimax-m3-msa-tech-report), section 核心机制:
 *   - 索引分支 (index branch): the token score equation S^idx and the block
 *     max-pool M^idx (scores of visible keys j <= i only), then the TopK
 *     equation per GQA group, with the query's own block always selected.
 *   - 主分支 (main branch): the softmax attention equation O^(h)_i over the
 *     selected blocks' visible tokens, all heads of a group sharing the group's
 *     selection.
 * and, for msa_oracle_kl, section 训练 of the same page: the index branch's
 * distribution P^idx and the group-averaged main-branch distribution P^(r) over
 * the selected tokens, and the alignment loss L_KL = KL(P^(r) || P^idx); and, for
 * msa_oracle_attn_bwd, the gradients of the main-branch equation with respect to q,
 * k and v for a given output gradient, the selection held fixed (the same section
 * cuts the index branch's gradient from the main branch); and, for msa_oracle_project,
 * the two projection matrices the index branch adds to GQA (section 核心机制, 索引分支):
 * one index query head per group and one index key shared by the groups.
 *
 * Readings where the page is silent (each is listed with its reason in the
 * design notes):
 *   - top_k counts the forced local block: the selection is the local block
 *     plus the best top_k-1 of the earlier blocks.
 *   - order of blocks: score descending, then block index ascending.
 *   - if the query sees top_k blocks or fewer, all of them are selected.
 *   - the selection is reported in ascending block order, padded with -1.
 *   - the positive factor 1/sqrt(d_idx) does not change the order, so block
 *     scores are reported as raw maxima of the dot products.
 *   - head h belongs to group h / (H_q / H_kv).
 *
 * Precision: every input element (fp32 or bf16 storage) is widened exactly to
 * double; all arithmetic is double; outputs are double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* storage type of an input array */
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* Widen element i of an fp32 or bf16 array to double, exactly. */
static double elem(const void *base, int64_t i, int type) {
  if (type == ORACLE_F32) return (double)((const float *)base)[i];
  uint32_t bits = ((uint32_t)((const uint16_t *)base)[i]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

typedef struct {
  double score;
  int32_t block;
} scored_block;

/* Order used by TopK: higher score first; equal scores -> lower block first. */
static int by_score_then_block(const void *a, const void *b) {
  const scored_block *x = (const scored_block *)a, *y = (const scored_block *)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->block > y->block) - (x->block < y->block);
}

static int ascending_int(const void *a, const void *b) {
  int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

/*
 * Index branch for one (sequence, group, query row) at absolute position p.
 *   q_idx_row : d_idx elements of this row's index query (group r)
 *   k_idx_seq : the sequence's shared index keys, row j at j*d_idx
 *   scores    : scratch of p+1 doubles
 *   bmax      : out, n_blocks doubles: raw block maxima, -inf past the local block
 *   sel       : out, top_k block indices ascending, -1 padded
 */
static void index_row(const void *q_idx_row, const void *k_idx_seq, int type, int d_idx,
                      int n_blocks, int64_t p, int block_size, int top_k, double *scores,
                      scored_block *cand, double *bmax, int32_t *sel) {
  /* token scores S_j = q_idx . k_idx_j for visible keys j <= p (the 1/sqrt(d_idx)
     factor is positive and left out) */
  for (int64_t j = 0; j <= p; ++j) {
    double s = 0.0;
    for (int d = 0; d < d_idx; ++d)
      s += elem(q_idx_row, d, type) * elem(k_idx_seq, j * d_idx + d, type);
    scores[j] = s;
  }
  /* causal block max-pool: block c covers keys [c*bs, (c+1)*bs), clipped at p */
  const int64_t local = p / block_size;
  for (int c = 0; c < n_blocks; ++c) {
    if (c > local) {
      bmax[c] = -INFINITY;
      continue;
    }
    int64_t lo = (int64_t)c * block_size, hi = lo + block_size;
    if (hi > p + 1) hi = p + 1;
    double m = -INFINITY;
    for (int64_t j = lo; j < hi; ++j)
      if (scores[j] > m) m = scores[j];
    bmax[c] = m;
  }
  /* TopK with the local block forced in */
  int n_sel = 0;
  if (local + 1 <= top_k) {
    for (int c = 0; c <= local; ++c) sel[n_sel++] = c;
  } else {
    for (int c = 0; c < local; ++c) {
      cand[c].score = bmax[c];
      cand[c].block = c;
    }
    qsort(cand, (size_t)local, sizeof(scored_block), by_score_then_block);
    for (int i = 0; i < top_k - 1; ++i) sel[n_sel++] = cand[i].block;
    sel[n_sel++] = (int32_t)local;
    qsort(sel, (size_t)n_sel, sizeof(int32_t), ascending_int);
  }
  for (int i = n_sel; i < top_k; ++i) sel[i] = -1;
}

/*
 * Main branch for one (sequence, head, query row) at position p:
 *   T = union over selected blocks c of the visible keys [c*bs, min((c+1)*bs, p+1))
 *   z_j = q . k_j / sqrt(d_h);  O = sum_j softmax(z)_j v_j;  lse = log sum_j exp(z_j)
 *   q_row : d_h elements; k_plane, v_plane : the group's keys/values, row j at j*d_h
 */
static void attend_row(const void *q_row, const void *k_plane, const void *v_plane, int type,
                       int d_h, int64_t p, int block_size, const int32_t *sel, int top_k,
                       double *z, double *o, double *lse) {
  const double scale = 1.0 / sqrt((double)d_h);
  int64_t n = 0;
  double mu = -INFINITY;
  for (int i = 0; i < top_k; ++i) {
    if (sel[i] < 0) continue;
    int64_t lo = (int64_t)sel[i] * block_size, hi = lo + block_size;
    if (hi > p + 1) hi = p + 1;
    for (int64_t j = lo; j < hi; ++j) {
      double s = 0.0;
      for (int d = 0; d < d_h; ++d) s += elem(q_row, d, type) * elem(k_plane, j * d_h + d, type);
      z[n] = s * scale;
      if (z[n] > mu) mu = z[n];
      ++n;
    }
  }
  for (int d = 0; d < d_h; ++d) o[d] = 0.0;
  double total = 0.0;
  n = 0;
  for (int i = 0; i < top_k; ++i) {
    if (sel[i] < 0) continue;
    int64_t lo = (int64_t)sel[i] * block_size, hi = lo + block_size;
    if (hi > p + 1) hi = p + 1;
    for (int64_t j = lo; j < hi; ++j) {
      double w = exp(z[n++] - mu);
      total += w;
      for (int d = 0; d < d_h; ++d) o[d] += w * elem(v_plane, j * d_h + d, type);
    }
  }
  for (int d = 0; d < d_h; ++d) o[d] /= total;
  *lse = mu + log(total);
}

/*
 * The whole MSA step for a list of query rows.
 *
 * Layouts (contiguous):
 *   q_idx [B, H_kv, n_q, d_idx]   k_idx [B, n_k, d_idx]
 *   q     [B, H_q,  n_q, d_h]     k, v  [B, H_kv, n_k, d_h]
 * rows[i] in [0, n_q) selects query row rows[i]; its position is q_start + rows[i].
 * Outputs (per listed row, in list order):
 *   sel   [B, H_kv, n_rows, top_k]            int32
 *   bmax  [B, H_kv, n_rows, n_blocks] or NULL double
 *   o     [B, H_q, n_rows, d_h] or NULL       double (NULL: index branch only)
 *   lse   [B, H_q, n_rows] or NULL            double
 * Returns 0, or -1 on a bad argument, -2 when out of memory.
 */
int msa_oracle_run(int batch, int n_q, int n_k, int q_start, int h_q, int h_kv, int d_h,
                   int d_idx, int block_size, int top_k, int type, const void *q_idx,
                   const void *k_idx, const void *q, const void *k, const void *v, int n_rows,
                   const int32_t *rows, int32_t *sel, double *bmax, double *o, double *lse,
                   int n_threads) {
  if (batch < 1 || n_q < 1 || n_k < 1 || q_start < 0 || h_kv < 1 || h_q < h_kv ||
      h_q % h_kv || d_idx < 1 || block_size < 1 || top_k < 1 || n_rows < 0 || !q_idx ||
      !k_idx || !rows || !sel || (type != ORACLE_F32 && type != ORACLE_BF16))
    return -1;
  if (o && (!q || !k || !v || d_h < 1)) return -1;
  for (int i = 0; i < n_rows; ++i)
    if (rows[i] < 0 || rows[i] >= n_q || (int64_t)q_start + rows[i] >= n_k) return -1;
  const int n_blocks = (n_k + block_size - 1) / block_size;
  const int group = h_q / h_kv;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
  int failed = 0;

  /* index branch: one task per (b, r, row) */
  const int64_t n_idx_tasks = (int64_t)batch * h_kv * n_rows;
#pragma omp parallel
  {
    double *scores = (double *)malloc(sizeof(double) * (size_t)n_k);
    double *bm = (double *)malloc(sizeof(double) * (size_t)n_blocks);
    scored_block *cand = (scored_block *)malloc(sizeof(scored_block) * (size_t)n_blocks);
    if (!scores || !bm || !cand) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t task = 0; task < n_idx_tasks; ++task) {
      if (failed) continue;
      const int i = (int)(task % n_rows);
      const int r = (int)((task / n_rows) % h_kv);
      const int b = (int)(task / ((int64_t)n_rows * h_kv));
      const int64_t t = rows[i], p = (int64_t)q_start + t;
      const int64_t qoff = (((int64_t)b * h_kv + r) * n_q + t) * d_idx;
      const int64_t koff = (int64_t)b * n_k * d_idx;
      const void *qrow = (type == ORACLE_F32) ? (const void *)((const float *)q_idx + qoff)
                                              : (const void *)((const uint16_t *)q_idx + qoff);
      const void *kseq = (type == ORACLE_F32) ? (const void *)((const float *)k_idx + koff)
                                              : (const void *)((const uint16_t *)k_idx + koff);
      const int64_t out = ((int64_t)b * h_kv + r) * n_rows + i;
      index_row(qrow, kseq, type, d_idx, n_blocks, p, block_size, top_k, scores, cand, bm,
                sel + out * top_k);
      if (bmax) memcpy(bmax + out * n_blocks, bm, sizeof(double) * (size_t)n_blocks);
    }
    free(scores);
    free(bm);
    free(cand);
  }
  if (failed) return -2;
  if (!o) return 0;

  /* main branch: one task per (b, h, row) */
  const int64_t n_att_tasks = (int64_t)batch * h_q * n_rows;
  const int64_t max_t = (int64_t)top_k * block_size;
#pragma omp parallel
  {
    double *z = (double *)malloc(sizeof(double) * (size_t)max_t);
    if (!z) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t task = 0; task < n_att_tasks; ++task) {
      if (failed) continue;
      const int i = (int)(task % n_rows);
      const int h = (int)((task / n_rows) % h_q);
      const int b = (int)(task / ((int64_t)n_rows * h_q));
      const int r = h / group;
      const int64_t t = rows[i], p = (int64_t)q_start + t;
      const int64_t qoff = (((int64_t)b * h_q + h) * n_q + t) * d_h;
      const int64_t kvoff = ((int64_t)b * h_kv + r) * (int64_t)n_k * d_h;
      const size_t es = (type == ORACLE_F32) ? 4 : 2;
      const void *qrow = (const char *)q + qoff * (int64_t)es;
      const void *kp = (const char *)k + kvoff * (int64_t)es;
      const void *vp = (const char *)v + kvoff * (int64_t)es;
      const int32_t *s = sel + (((int64_t)b * h_kv + r) * n_rows + i) * top_k;
      const int64_t out = ((int64_t)b * h_q + h) * n_rows + i;
      double l;
      attend_row(qrow, kp, vp, type, d_h, p, block_size, s, top_k, z, o + out * d_h, &l);
      if (lse) lse[out] = l;
    }
    free(z);
  }
  return failed ? -2 : 0;
}

/*
 * Alignment loss for one (sequence, group r, query row) at position p, given the row's
 * selection (section 训练: the equations for P^idx, P^(r) and L_KL):
 *   T          = the selected blocks' visible tokens (the main branch's token set)
 *   S^idx_j    = q_idx . k_idx_j / sqrt(d_idx)       P^idx = softmax over T of S^idx
 *   S^(l)_j    = q_l . k_j / sqrt(d_h), l in group r P^(r) = (1/G) sum_l softmax_T(S^(l))
 *   L_KL       = sum_{j in T} P^(r)_j (log P^(r)_j - log P^idx_j), natural log; a term
 *                with P^(r)_j = 0 adds 0.
 *   lse_idx    = log sum_{j in T} exp(S^idx_j), the normaliser of P^idx.
 * q_row0: the group's first query row, head l at l * q_head_stride elements; k_plane: the
 * group's keys. Scratch (top_k * block_size each): key, sidx, zh, t.
 */
static void kl_row(const void *q_idx_row, const void *k_idx_seq, const void *q_row0,
                   int64_t q_head_stride, const void *k_plane, int type, int d_idx, int d_h,
                   int group, int64_t p, int block_size, const int32_t *sel, int top_k,
                   int64_t *key, double *sidx, double *zh, double *t, double *kl,
                   double *lse_idx) {
  const size_t es = (type == ORACLE_F32) ? 4 : 2;
  /* the token set T and the index scores S^idx on it */
  int64_t n = 0;
  for (int i = 0; i < top_k; ++i) {
    if (sel[i] < 0) continue;
    int64_t lo = (int64_t)sel[i] * block_size, hi = lo + block_size;
    if (hi > p + 1) hi = p + 1;
    for (int64_t j = lo; j < hi; ++j) {
      double s = 0.0;
      for (int d = 0; d < d_idx; ++d)
        s += elem(q_idx_row, d, type) * elem(k_idx_seq, j * d_idx + d, type);
      key[n] = j;
      sidx[n] = s / sqrt((double)d_idx);
      ++n;
    }
  }
  /* student: log P^idx_j = S^idx_j - lse_idx */
  double mu = -INFINITY;
  for (int64_t j = 0; j < n; ++j)
    if (sidx[j] > mu) mu = sidx[j];
  double zsum = 0.0;
  for (int64_t j = 0; j < n; ++j) zsum += exp(sidx[j] - mu);
  const double lse_s = mu + log(zsum);
  /* teacher: P^(r)_j = mean over the group's heads l of softmax_T(S^(l))_j */
  for (int64_t j = 0; j < n; ++j) t[j] = 0.0;
  const double scale = 1.0 / sqrt((double)d_h);
  for (int l = 0; l < group; ++l) {
    const void *q_row = (const char *)q_row0 + (int64_t)l * q_head_stride * (int64_t)es;
    double hm = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
      double s = 0.0;
      for (int d = 0; d < d_h; ++d) s += elem(q_row, d, type) * elem(k_plane, key[j] * d_h + d, type);
      zh[j] = s * scale;
      if (zh[j] > hm) hm = zh[j];
    }
    double hs = 0.0;
    for (int64_t j = 0; j < n; ++j) hs += exp(zh[j] - hm);
    for (int64_t j = 0; j < n; ++j) t[j] += exp(zh[j] - hm) / hs / (double)group;
  }
  /* L_KL = sum_j P^(r)_j (log P^(r)_j - log P^idx_j) */
  double loss = 0.0;
  for (int64_t j = 0; j < n; ++j)
    if (t[j] > 0.0) loss += t[j] * (log(t[j]) - (sidx[j] - lse_s));
  *kl = loss;
  *lse_idx = lse_s;
}

/*
 * The alignment loss for a list of query rows, given their selections.
 *   sel [B, H_kv, n_rows, top_k] (as msa_oracle_run writes it for the same rows)
 *   kl, lse_idx [B, H_kv, n_rows] double (lse_idx may be NULL)
 * Layouts of q_idx, k_idx, q, k as for msa_oracle_run. Returns 0, -1 on a bad argument,
 * -2 when out of memory.
 */
int msa_oracle_kl(int batch, int n_q, int n_k, int q_start, int h_q, int h_kv, int d_h,
                  int d_idx, int block_size, int top_k, int type, const void *q_idx,
                  const void *k_idx, const void *q, const void *k, int n_rows,
                  const int32_t *rows, const int32_t *sel, double *kl, double *lse_idx,
                  int n_threads) {
  if (batch < 1 || n_q < 1 || n_k < 1 || q_start < 0 || h_kv < 1 || h_q < h_kv ||
      h_q % h_kv || d_idx < 1 || d_h < 1 || block_size < 1 || top_k < 1 || n_rows < 0 ||
      !q_idx || !k_idx || !q || !k || !rows || !sel || !kl ||
      (type != ORACLE_F32 && type != ORACLE_BF16))
    return -1;
  for (int i = 0; i < n_rows; ++i)
    if (rows[i] < 0 || rows[i] >= n_q || (int64_t)q_start + rows[i] >= n_k) return -1;
  const int group = h_q / h_kv;
  const size_t es = (type == ORACLE_F32) ? 4 : 2;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
  int failed = 0;
  const int64_t n_tasks = (int64_t)batch * h_kv * n_rows;
  const int64_t max_t = (int64_t)top_k * block_size;
#pragma omp parallel
  {
    int64_t *key = (int64_t *)malloc(sizeof(int64_t) * (size_t)max_t);
    double *sidx = (double *)malloc(sizeof(double) * (size_t)max_t);
    double *zh = (double *)malloc(sizeof(double) * (size_t)max_t);
    double *t = (double *)malloc(sizeof(double) * (size_t)max_t);
    if (!key || !sidx || !zh || !t) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t task = 0; task < n_tasks; ++task) {
      if (failed) continue;
      const int i = (int)(task % n_rows);
      const int r = (int)((task / n_rows) % h_kv);
      const int b = (int)(task / ((int64_t)n_rows * h_kv));
      const int64_t tq = rows[i], p = (int64_t)q_start + tq;
      const int64_t qi_off = (((int64_t)b * h_kv + r) * n_q + tq) * d_idx;
      const int64_t ki_off = (int64_t)b * n_k * d_idx;
      const int64_t q_off = (((int64_t)b * h_q + (int64_t)r * group) * n_q + tq) * d_h;
      const int64_t k_off = ((int64_t)b * h_kv + r) * (int64_t)n_k * d_h;
      const int64_t out = ((int64_t)b * h_kv + r) * n_rows + i;
      double l;
      kl_row((const char *)q_idx + qi_off * (int64_t)es, (const char *)k_idx + ki_off * (int64_t)es,
             (const char *)q + q_off * (int64_t)es, (int64_t)n_q * d_h,
             (const char *)k + k_off * (int64_t)es, type, d_idx, d_h, group, p, block_size,
             sel + out * top_k, top_k, key, sidx, zh, t, kl + out, &l);
      if (lse_idx) lse_idx[out] = l;
    }
    free(key);
    free(sidx);
    free(zh);
    free(t);
  }
  return failed ? -2 : 0;
}

/*
 * Gradient of the main branch for one (sequence, head, row) at position p, accumulated:
 *   z_j = q . k_j / sqrt(d_h),  P = softmax_T(z),  O = sum_j P_j v_j  (T as for attend_row)
 *   for an output gradient dO:  dv_j += P_j dO
 *                               dP_j = dO . v_j,  dz_j = P_j (dP_j - sum_u P_u dP_u)
 *                               dq   += sum_j dz_j k_j / sqrt(d_h)
 *                               dk_j += dz_j q / sqrt(d_h)
 * dq: d_h doubles for this (head, row); dk, dv: the group's planes [n_k, d_h].
 */
static void attend_row_bwd(const void *q_row, const void *k_plane, const void *v_plane,
                           const void *do_row, int type, int d_h, int64_t p, int block_size,
                           const int32_t *sel, int top_k, int64_t *key, double *z,
                           double *dp, double *dq, double *dk, double *dv) {
  const double scale = 1.0 / sqrt((double)d_h);
  int64_t n = 0;
  double mu = -INFINITY;
  for (int i = 0; i < top_k; ++i) {
    if (sel[i] < 0) continue;
    int64_t lo = (int64_t)sel[i] * block_size, hi = lo + block_size;
    if (hi > p + 1) hi = p + 1;
    for (int64_t j = lo; j < hi; ++j) {
      double s = 0.0;
      for (int d = 0; d < d_h; ++d) s += elem(q_row, d, type) * elem(k_plane, j * d_h + d, type);
      key[n] = j;
      z[n] = s * scale;
      if (z[n] > mu) mu = z[n];
      ++n;
    }
  }
  double total = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    z[j] = exp(z[j] - mu);
    total += z[j];
  }
  double dsum = 0.0; /* sum_u P_u dP_u */
  for (int64_t j = 0; j < n; ++j) {
    z[j] /= total; /* P_j */
    double s = 0.0;
    for (int d = 0; d < d_h; ++d) s += elem(do_row, d, type) * elem(v_plane, key[j] * d_h + d, type);
    dp[j] = s;
    dsum += z[j] * s;
  }
  for (int64_t j = 0; j < n; ++j) {
    const double dz = z[j] * (dp[j] - dsum);
    for (int d = 0; d < d_h; ++d) {
      dq[d] += dz * elem(k_plane, key[j] * d_h + d, type) * scale;
      dk[key[j] * d_h + d] += dz * elem(q_row, d, type) * scale;
      dv[key[j] * d_h + d] += z[j] * elem(do_row, d, type);
    }
  }
}

/*
 * Main-branch gradients for every row of every sequence, given the selections.
 *   q, k, v and sel as for msa_oracle_run (sel [B, H_kv, n_q, top_k], all rows);
 *   dout [B, H_q, n_q, d_h] in the storage type of the inputs.
 *   dq [B, H_q, n_q, d_h], dk and dv [B, H_kv, n_k, d_h]: double, overwritten.
 * One task per (sequence, group): it owns that group's dk and dv planes.
 * Returns 0, -1 on a bad argument, -2 when out of memory.
 */
int msa_oracle_attn_bwd(int batch, int n_q, int n_k, int q_start, int h_q, int h_kv, int d_h,
                        int block_size, int top_k, int type, const void *q, const void *k,
                        const void *v, const int32_t *sel, const void *dout, double *dq,
                        double *dk, double *dv, int n_threads) {
  if (batch < 1 || n_q < 1 || n_k < 1 || q_start < 0 || h_kv < 1 || h_q < h_kv ||
      h_q % h_kv || d_h < 1 || block_size < 1 || top_k < 1 || (int64_t)q_start + n_q > n_k ||
      !q || !k || !v || !sel || !dout || !dq || !dk || !dv ||
      (type != ORACLE_F32 && type != ORACLE_BF16))
    return -1;
  const int group = h_q / h_kv;
  const size_t es = (type == ORACLE_F32) ? 4 : 2;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
  memset(dq, 0, sizeof(double) * (size_t)batch * h_q * n_q * d_h);
  memset(dk, 0, sizeof(double) * (size_t)batch * h_kv * n_k * d_h);
  memset(dv, 0, sizeof(double) * (size_t)batch * h_kv * n_k * d_h);
  int failed = 0;
  const int64_t max_t = (int64_t)top_k * block_size;
#pragma omp parallel
  {
    int64_t *key = (int64_t *)malloc(sizeof(int64_t) * (size_t)max_t);
    double *z = (double *)malloc(sizeof(double) * (size_t)max_t);
    double *dp = (double *)malloc(sizeof(double) * (size_t)max_t);
    if (!key || !z || !dp) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t task = 0; task < (int64_t)batch * h_kv; ++task) {
      if (failed) continue;
      const int r = (int)(task % h_kv), b = (int)(task / h_kv);
      const int64_t kv_off = ((int64_t)b * h_kv + r) * (int64_t)n_k * d_h;
      const void *kp = (const char *)k + kv_off * (int64_t)es;
      const void *vp = (const char *)v + kv_off * (int64_t)es;
      for (int l = 0; l < group; ++l) {
        const int h = r * group + l;
        for (int t = 0; t < n_q; ++t) {
          const int64_t row = ((int64_t)b * h_q + h) * n_q + t;
          attend_row_bwd((const char *)q + row * d_h * (int64_t)es, kp, vp,
                         (const char *)dout + row * d_h * (int64_t)es, type, d_h,
                         (int64_t)q_start + t, block_size,
                         sel + (((int64_t)b * h_kv + r) * n_q + t) * top_k, top_k, key, z, dp,
                         dq + row * d_h, dk + kv_off, dv + kv_off);
        }
      }
    }
    free(key);
    free(z);
    free(dp);
  }
  return failed ? -2 : 0;
}

/*
 * Index-branch projections of the hidden states x, one output element at a time:
 *   q_idx[b, r, t, d] = sum_i x[b, t, i] * w_q[r * d_idx + d, i]   (one head per group r)
 *   k_idx[b, t, d]    = sum_i x[b, t, i] * w_k[d, i]               (shared by the groups)
 * x [B, n, d_model], w_q [h_kv * d_idx, d_model] and w_k [d_idx, d_model] in the storage
 * type (each weight row holds one output's coefficients); q_idx [B, h_kv, n, d_idx] and
 * k_idx [B, n, d_idx] double, overwritten. Returns 0, or -1 on a bad argument.
 */
int msa_oracle_project(int batch, int n, int d_model, int h_kv, int d_idx, int type,
                       const void *x, const void *w_q, const void *w_k, double *q_idx,
                       double *k_idx, int n_threads) {
  if (batch < 1 || n < 1 || d_model < 1 || h_kv < 1 || d_idx < 1 || !x || !w_q || !w_k ||
      !q_idx || !k_idx || (type != ORACLE_F32 && type != ORACLE_BF16))
    return -1;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
#pragma omp parallel for schedule(static)
  for (int64_t row = 0; row < (int64_t)batch * n; ++row) {
    const int64_t b = row / n, t = row % n;
    const int64_t xo = row * d_model;
    for (int r = 0; r < h_kv; ++r)
      for (int d = 0; d < d_idx; ++d) {
        const int64_t wo = ((int64_t)r * d_idx + d) * d_model;
        double s = 0.0;
        for (int i = 0; i < d_model; ++i) s += elem(x, xo + i, type) * elem(w_q, wo + i, type);
        q_idx[((b * h_kv + r) * n + t) * d_idx + d] = s;
      }
    for (int d = 0; d < d_idx; ++d) {
      double s = 0.0;
      for (int i = 0; i < d_model; ++i)
        s += elem(x, xo + i, type) * elem(w_k, (int64_t)d * d_model + i, type);
      k_idx[row * d_idx + d] = s;
    }
  }
  return 0;
}

/* Threads the oracle will use when n_threads <= 0. */
int msa_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
