// msa_index.hip -- index branch: token scores q_idx . k_idx on the matrix cores with the
// causal block max-pool fused into the epilogue.
//
// Definition ("MiniMax-M3: MSA 技术报告速读", section 核心机制, index-branch score and
// max-pool equation): M[b,r,t,c] = max over keys j of block c with j <= p(t) of
// q_idx[b,r,t,:] . k_idx[b,j,:]. The 1/sqrt(d_idx) factor is positive and left out.
//
// The product is computed transposed, S^T = K_idx * Q_idx^T, so that the keys of a block
// run down the accumulator rows each lane holds: pooling is an in-lane max over the
// lane's rows followed by two lane-group swaps, not a shuffle reduction over keys.
#include "msa_device.hpp"
#include "msa_internal.hpp"
#include "msa_select.hpp"

#include <type_traits>

namespace msa {
namespace {

constexpr int KT = 64;        // keys per key tile: four 16-row MFMA tiles
constexpr int SEL_WAVES = 8;  // waves of a decode index-select workgroup
constexpr int WG_COLS = 256;  // (group, query) columns per prefill workgroup: 4 waves x 64

template <typename E, int DI>
struct KTile {
  static constexpr bool SWZ = sizeof(E) == 2;  // a matrix-core fragment is one 16-byte piece
  static constexpr int ROW = DI * (int)sizeof(E) + (SWZ ? 0 : 16);  // LDS row (bytes)
  static constexpr int PER_ROW = DI * (int)sizeof(E) / 16;      // 16-byte pieces per key
  // Byte offset of a key's 16-byte piece. For 2-byte elements the piece index is XORed
  // with the key's low bits: the fragment reads (16 keys at one piece per 16 lanes) are
  // then free of bank conflicts, where rows padded by 16 bytes averaged 2.8 conflict
  // cycles per LDS instruction (SQ_LDS_BANK_CONFLICT) and padding by 32 bytes lost a
  // workgroup per CU. An fp32 fragment spans two pieces, kept adjacent in padded rows.
  static __device__ __forceinline__ int at(int key, int piece) {
    if constexpr (SWZ)
      return key * ROW + (piece ^ (key & (PER_ROW - 1))) * 16;
    else
      return key * ROW + piece * 16;
  }
  static constexpr int PIECES = KT * PER_ROW;
  static constexpr int PER_THREAD = PIECES / 256;
};

__global__ void fill_kernel(float *p, size_t n, float value) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = value;
}

// Prefill / chunked prefill. Grid: x = query tile, y = key chunk, z = sequence. The query
// tile varies fastest so that consecutive workgroups, which the dispatcher deals round-robin
// to the eight XCDs, have the same amount of causal work: with the key chunk fastest, the
// XCD would be fixed by the chunk index and the early chunks (present in every row) would
// pile onto a few XCDs. Workgroups on one XCD then also share the chunk's k_idx in L2.
// A workgroup owns TQ = 256 / R query rows for all R groups (256 columns; wave w takes
// columns 64w..64w+63 as four 16-column N-tiles) and one chunk of keys. The k_idx tile
// is staged once in LDS (double-buffered) and feeds every group: the index key is shared.
// Pooled maxima are collected in LDS for OUT_RUN consecutive blocks and written as
// contiguous runs of each output row. With RK, each lane also keeps the largest maximum of
// its column over the run and writes its order key as the run's key (key chunks are then
// whole runs, so runs are aligned: blocks 32 r .. 32 r + 31).
constexpr int OUT_RUN = RUN_BLOCKS;

// bf16 asks the compiler for three waves per SIMD; fp32 (twice the fragment registers)
// cannot fit three and takes the default.
template <typename E, int DI, int BS, bool RK, bool CF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(E) == 2 ? 3 : 1)))
void index_pool_prefill(IndexArgs a) {
  using L = KTile<E, DI>;
  using F = typename Frag<E>::type;
  constexpr int DC = DI / 32;
  constexpr int BPT = KT / BS;  // blocks per key tile
  constexpr int MPB = BS / 16;  // 16-key row tiles per block
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][KT * L::ROW];
  __shared__ float s_out[WG_COLS][OUT_RUN + 1];  // padded: conflict-free column writes

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int R = a.h_kv, TQ = WG_COLS / R;
  const int b = blockIdx.z;
  const int t0 = blockIdx.x * TQ;
  const int t_last = min(t0 + TQ, a.n_q) - 1;
  const long p_first = (long)a.q_start + t0, p_last = (long)a.q_start + t_last;
  const long k_begin = (long)blockIdx.y * a.key_chunk;
  if (k_begin > p_last) return;  // uniform over the workgroup
  const long k_end = min(k_begin + (long)a.key_chunk, p_last + 1);
  const int n_tiles = (int)((k_end - k_begin + KT - 1) / KT);
  const long c_begin = k_begin / BS;  // first block of the chunk (a multiple of OUT_RUN with RK)

  // B operand: q_idx of this lane's four columns (column = lane % 16 of each N-tile).
  const E *qi = reinterpret_cast<const E *>(a.q_idx);
  F bq[4][DC];
  int prel[4];  // column position minus the chunk's first key (clamped to int range)
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int col = w * 64 + nt * 16 + c16, r = col / TQ, t = t0 + col % TQ;
    prel[nt] = (int)min((long)a.q_start + t - k_begin, (long)0x3fffffff);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      bq[nt][dc] = (t < a.n_q)
                       ? load_frag(qi + (((long)b * R + r) * a.n_q + t) * DI + dc * 32 + g * 8)
                       : zero_frag(qi);
  }

  const unsigned char *kbase =
      reinterpret_cast<const unsigned char *>(a.k_idx) + (long)b * a.cap * DI * (long)sizeof(E);
  // k_idx tiles arrive two tiles ahead: tile j's pieces load into register set j % 2 while
  // tiles j-2 and j-1 compute, and are stashed into LDS buffer j % 2 after tile j-1.
  u32x4 pa[L::PER_THREAD], pb[L::PER_THREAD];
  // Keys past n_k read key n_k - 1 instead: they lie past every column's position, so the
  // pooling masks them, and an unconditional load keeps the compiler's waits precise.
  auto fetch = [&](int tile, u32x4 (&pre)[L::PER_THREAD]) {
    const long k0 = k_begin + (long)tile * KT;
#pragma unroll
    for (int i = 0; i < L::PER_THREAD; ++i) {
      const int pc = tid + i * 256, key = pc / L::PER_ROW, off = pc % L::PER_ROW;
      const long j = min(k0 + key, (long)a.n_k - 1);
      pre[i] = *reinterpret_cast<const u32x4 *>(kbase + j * DI * (long)sizeof(E) + off * 16);
    }
  };
  auto stash = [&](int buf, const u32x4 (&pre)[L::PER_THREAD]) {
#pragma unroll
    for (int i = 0; i < L::PER_THREAD; ++i) {
      const int pc = tid + i * 256, key = pc / L::PER_ROW, off = pc % L::PER_ROW;
      *reinterpret_cast<u32x4 *>(&lds[buf][L::at(key, off)]) = pre[i];
    }
  };
  // Write s_out's first n blocks of every column to block columns [c0, c0 + n) of the rows:
  // OUT_RUN / 4 threads per column, four blocks each.
  auto flush = [&](long c0, int n) {
    constexpr int TPC = OUT_RUN / 4;
    const int j0 = (tid % TPC) * 4;
    for (int col = tid / TPC; col < WG_COLS; col += 256 / TPC) {
      const int r = col / TQ, t = t0 + col % TQ;
      if (t >= a.n_q) continue;
      const long base = (((long)b * R + r) * a.n_q + t) * (long)a.n_blocks + c0;
      if (n >= j0 + 4 && c0 + j0 + 4 <= a.n_blocks && ((base + j0) & 3) == 0) {
        *reinterpret_cast<f32x4 *>(a.bmax + base + j0) =
            f32x4{s_out[col][j0], s_out[col][j0 + 1], s_out[col][j0 + 2], s_out[col][j0 + 3]};
      } else {
        for (int j = j0; j < min(n, j0 + 4); ++j)
          if (c0 + j < a.n_blocks) a.bmax[base + j] = s_out[col][j];
      }
    }
  };

  // CF (rows a whole number of runs long, runs aligned, a spare destination given): each
  // wave writes its own 64 columns' run, 8 lanes per column and 16 bytes per lane, always 8
  // stores per lane with no branch. Blocks past the run's end are written as -inf, their
  // value: they lie past every row's local block (the run ends where the last row's keys
  // do) and inside the row. Columns past the rows write the spare 16 bytes. The compiler
  // counts these stores, so no wait for them follows, and no barrier either: only this
  // wave's lanes wrote these columns of s_out and only they read them.
  auto flush_counted = [&](long c0, int n) {
    // The lane index as the asm leaves it: the addresses below are then computed here, not
    // hoisted out of the tile loop into registers held all along.
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int pc = ln + 64 * i, col = w * 64 + (pc >> 3), j0 = (pc & 7) * 4;
      const int r = col / TQ, t = t0 + col % TQ;
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = s_out[col][j0 + e];  // every lane reads, then selects
#pragma unroll
      for (int e = 0; e < 4; ++e) pin(x[e]);
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = j0 + e < n ? x[e] : -INFINITY;
      float *dst = t < a.n_q ? a.bmax + (((long)b * R + r) * a.n_q + t) * a.n_blocks + c0 + j0
                             : a.spare;
      *reinterpret_cast<f32x4 *>(dst) = v;
      // one store at a time: hoisting every piece's reads and address ahead of the stores
      // took the registers of the main loop
      asm volatile("" ::: "memory");
    }
  };

  const int my_col = w * 64 + g * 16 + c16;  // the column whose pooled value this lane holds
  int run = 0;  // blocks collected in s_out
  float rk = -INFINITY;  // RK: largest maximum of my_col's blocks in the current run
  // One key tile: pooled maxima of LDS buffer `buf` into s_out, the next tile's pieces
  // (register set `nxt`, loaded a tile earlier) into the other buffer, and the flush of a
  // full run of blocks.
  auto tile_step = [&](int tile, u32x4 (&nxt)[L::PER_THREAD]) {
    const int buf = tile & 1;
    const long k0 = k_begin + (long)tile * KT;
    const int krel = tile * KT;  // k0 - k_begin
    const bool need_mask = k0 + KT - 1 > p_first;

    F af[4][DC];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        af[mt][dc] = load_frag(reinterpret_cast<const E *>(
            &lds[buf][L::at(mt * 16 + c16, (dc * 32 + g * 8) * (int)sizeof(E) / 16)]));
    f32x4 acc[4][4];  // [mt][nt]: S^T tile of 16 keys x 16 columns
    // A wave issuing its matrix-core chain goes first: the compute unit's other waves are
    // at their pooling, staging or barrier, and an idle matrix core costs more than a
    // delayed VALU or LDS instruction (the index kernel, 3.21 -> 3.15 ms at 128K, 3.09 ->
    // 2.95 ms on the 1M-context chunk; over the fragment reads and the pooling as well it
    // measured slower).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) c = mfma_chunk(af[mt][dc], bq[nt][dc], c);
        acc[mt][nt] = c;
      }
    __builtin_amdgcn_s_setprio(0);
    // Pool each block: max over its keys (rows), then over the four lane groups.
    auto pool = [&](auto masked) {
#pragma unroll
      for (int blk = 0; blk < BPT; ++blk) {
        float m[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          float v[4 * MPB];
#pragma unroll
          for (int mm = 0; mm < MPB; ++mm) {
            const int mt = blk * MPB + mm;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[mm * 4 + i] = acc[mt][nt][i];
            if constexpr (decltype(masked)::value) {
              // key offset (mt*16 + g*4 + i) is visible iff it is <= lim
              const int lim = prel[nt] - krel - (mt * 16 + g * 4);
#pragma unroll
              for (int i = 0; i < 4; ++i) v[mm * 4 + i] = (i <= lim) ? v[mm * 4 + i] : -INFINITY;
            }
          }
          m[nt] = max_chain<4 * MPB>(v);
        }
        const float pv = max_groups_transpose(m[0], m[1], m[2], m[3]);
        s_out[my_col][run + blk] = pv;
        if constexpr (RK) rk = fmaxf(rk, pv);
      }
    };
    if (need_mask)
      pool(std::true_type{});
    else
      pool(std::false_type{});
    run += BPT;
    if (tile + 1 < n_tiles) stash(buf ^ 1, nxt);
    __syncthreads();
    // This set is free again: tile + 3 goes into it (two tiles ahead of its stash). Past
    // the last tile the loads re-read it (cache hits): unconditional loads let the
    // compiler wait for exactly the set it stashes, not for every load in flight. With the
    // counted flush the loads go first, so that the set's registers are live across the
    // flush and are not reused for its stores (which would make the loads wait for them).
    if constexpr (CF) fetch(min(tile + 3, n_tiles - 1), nxt);
    if (run == OUT_RUN || tile + 1 == n_tiles) {
      const long c0 = c_begin + (long)(tile + 1) * BPT - run;
      if constexpr (CF) {
        flush_counted(c0, run);
      } else {
        flush(c0, run);
        // Wait for the maxima stores here, once per run: with stores of unknown completion
        // in flight the compiler makes every later wait for a k_idx tile a wait for all
        // memory operations (loads and stores need not complete in order), which would
        // also wait for the tile loaded a step later and undo the two-tile distance.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
      }
      run = 0;
      if constexpr (RK) {
        // One store per lane, after the maxima and with no branch (columns past the rows
        // write the spare word after the array), so the compiler counts it and the next
        // tiles' waits leave it in flight.
        const int r = my_col / TQ, t = t0 + my_col % TQ;
        const long at = t < a.n_q ? (((long)b * R + r) * a.n_q + t) * a.n_runs + c0 / OUT_RUN
                                  : (long)a.batch * R * a.n_q * a.n_runs;
        a.rkey[at] = order_key(rk);
        rk = -INFINITY;
      }
    }
    if constexpr (!CF) fetch(min(tile + 3, n_tiles - 1), nxt);
  };
  fetch(0, pa);
  fetch(min(1, n_tiles - 1), pb);
  stash(0, pa);
  fetch(min(2, n_tiles - 1), pa);
  __syncthreads();
  for (int tile = 0; tile < n_tiles; tile += 2) {
    tile_step(tile, pb);  // stashes tile + 1 from pb, then loads tile + 3 into pb
    if (tile + 1 < n_tiles) tile_step(tile + 1, pa);  // stashes tile + 2, loads tile + 4
  }
}

// Decode: one query row per sequence (all R groups in one 16-column N-tile). Each wave
// streams its own run of keys straight from HBM; the sequence's keys are split over many
// workgroups so the stream fills the chip. Grid: x = key chunk, z = sequence.
template <typename E, int DI, int BS>
__global__ __launch_bounds__(256) void index_pool_decode(IndexArgs a) {
  using F = typename Frag<E>::type;
  constexpr int DC = DI / 32;
  constexpr int BPT = KT / BS;
  constexpr int MPB = BS / 16;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int R = a.h_kv, b = blockIdx.z;
  const long p = a.q_start;
  const int sub = a.key_chunk / 4;
  const long k_begin = (long)blockIdx.x * a.key_chunk + (long)w * sub;
  if (k_begin > p) return;  // per wave; this kernel has no barrier
  const long k_end = min(k_begin + (long)sub, p + 1);

  const E *qi = reinterpret_cast<const E *>(a.q_idx);
  const E *ki = reinterpret_cast<const E *>(a.k_idx) + (long)b * a.cap * DI;
  F bq[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
    bq[dc] = (c16 < R) ? load_frag(qi + (((long)b * R + c16) * a.n_q) * DI + dc * 32 + g * 8)
                       : zero_frag(qi);
  float *out_row = a.bmax + ((long)b * R + c16) * a.n_q * (long)a.n_blocks;

  for (long k0 = k_begin; k0 < k_end; k0 += KT) {
    F af[4][DC];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const long j = k0 + mt * 16 + c16;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        af[mt][dc] = (j < a.n_k) ? load_frag(ki + j * DI + dc * 32 + g * 8) : zero_frag(ki);
    }
    const bool need_mask = k0 + KT - 1 > p;
#pragma unroll
    for (int blk = 0; blk < BPT; ++blk) {
      float m = -INFINITY;
#pragma unroll
      for (int mm = 0; mm < MPB; ++mm) {
        const int mt = blk * MPB + mm;
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) c = mfma_chunk(af[mt][dc], bq[dc], c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float s = c[i];
          if (need_mask && k0 + mt * 16 + g * 4 + i > p) s = -INFINITY;
          m = fmaxf(m, s);
        }
      }
      m = max_groups(m);
      const long cb = k0 / BS + blk;
      if (g == 0 && c16 < R && cb < a.n_blocks) out_row[cb] = m;
    }
  }
}

// Decode with the first selection stage fused in. Grid: x = range of SEL_NBLK key blocks,
// z = sequence; SEL_WAVES waves. Each wave pools its share of the blocks for all groups
// into LDS; then one wave per group ranks the range's blocks before the local block and
// writes its best top_k - 1 (key, block) pairs; a final merge pass picks the overall best.
//
// The k_idx stream is read once, so its loads are non-temporal; that only pays when every
// load instruction covers whole cache lines (a 512 MiB stream in this launch shape: 6.8 TB/s
// against 5.9 TB/s with ordinary loads, while non-temporal loads of the matrix-core
// fragment pattern, 64 bytes of each of 16 rows per instruction, made the kernel slower).
// So each 64-key tile is read as contiguous 1 KiB pieces, one 16-byte piece per lane, into
// registers a tile ahead, written to a wave-private LDS tile and read back as fragments.
//
// A fragment read's 16 lanes of one LDS pass take keys 0-7 at piece p and keys 8-15 at
// piece p + 1. bf16 rows of 128 bytes stay unpadded with the piece XORed by key & 7, which
// puts those 16 on distinct bank groups (rows padded by 16 bytes measured 3.8 conflict
// cycles per read); other rows keep 16 bytes of padding.
template <typename E, int DI>
struct SelStage {
  static constexpr int RB = DI * (int)sizeof(E);  // bytes of one key row
  static constexpr int PPK = RB / 16;             // 16-byte pieces per key
  static constexpr int PPL = KT * PPK / 64;       // pieces per lane and tile
  static constexpr bool SWZ = sizeof(E) == 2 && RB == 128;
  static constexpr int ROW = SWZ ? RB : RB + 16;
  static constexpr int WAVE_BYTES = KT * ROW;
  // byte offset of 16-byte piece `piece` of staged key `key`
  __device__ static __forceinline__ int at(int key, int piece) {
    return key * ROW + (SWZ ? piece ^ (key & 7) : piece) * 16;
  }
};

template <typename E, int DI, int BS>
__global__ __launch_bounds__(SEL_WAVES * 64) void index_select_decode(IndexArgs a) {
  using F = typename Frag<E>::type;
  using ST = SelStage<E, DI>;
  constexpr int DC = DI / 32;
  constexpr int BPT = KT / BS;
  constexpr int MPB = BS / 16;
  constexpr int NTW = SEL_NBLK * BS / KT;    // key tiles of the workgroup's range
  constexpr int SEL_BYTES = SEL_WAVES * SELECT_LDS * 8;
  constexpr int RAW = SEL_WAVES * ST::WAVE_BYTES > SEL_BYTES ? SEL_WAVES * ST::WAVE_BYTES : SEL_BYTES;
  __shared__ float s_m[16][SEL_NBLK];
  // the stream's staging tiles, then (after the barrier) the ranking's scratch
  __shared__ __attribute__((aligned(16))) unsigned char s_raw[RAW];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int R = a.h_kv, b = blockIdx.z, wg = blockIdx.x;
  const long p = a.q_start;
  const int local = (int)(p / BS);
  const int c0 = wg * SEL_NBLK;

  __shared__ int s_next;  // the range's next unclaimed key tile
  for (int x = tid; x < 16 * SEL_NBLK; x += SEL_WAVES * 64) (&s_m[0][0])[x] = -INFINITY;
  if (tid == 0) s_next = SEL_WAVES;  // tiles 0 .. SEL_WAVES-1 are the waves' first
  // counters of the kernel that follows in the same decode step start at zero
  if (wg == 0 && b == 0)
    for (int x = tid; x < a.n_zero; x += SEL_WAVES * 64) a.zero[x] = 0;
  __syncthreads();

  const E *qi = reinterpret_cast<const E *>(a.q_idx);
  const E *ki = reinterpret_cast<const E *>(a.k_idx) + (long)b * a.cap * DI;
  F bq[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
    bq[dc] = (c16 < R) ? load_frag(qi + (((long)b * R + c16) * a.n_q) * DI + dc * 32 + g * 8)
                       : zero_frag(qi);
  const long kb0 = (long)c0 * BS;  // the range's first key
  unsigned char *stg = s_raw + w * ST::WAVE_BYTES;
  // Keys past p read key p instead (pool masks them): unconditional loads keep the next
  // tile's loads in flight, where a load under a branch would make the MFMAs wait for all.
  auto fetch = [&](int tile, u32x4 (&dst)[ST::PPL]) {
    const long k0 = kb0 + (long)tile * KT;
#pragma unroll
    for (int i = 0; i < ST::PPL; ++i) {
      const int pc = i * 64 + lane;
      const long j = min(k0 + pc / ST::PPK, p);
      dst[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
          reinterpret_cast<const unsigned char *>(ki + j * DI) + (pc % ST::PPK) * 16));
    }
  };
  auto pool = [&](int tile, const u32x4 (&src)[ST::PPL]) {
    const long k0 = kb0 + (long)tile * KT;
    asm volatile("" ::: "memory");  // the previous tile's fragment reads come first
#pragma unroll
    for (int i = 0; i < ST::PPL; ++i) {
      const int pc = i * 64 + lane;
      *reinterpret_cast<u32x4 *>(stg + ST::at(pc / ST::PPK, pc % ST::PPK)) = src[i];
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // wave-private tile: in-order LDS
    F cur[4][DC];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        cur[mt][dc] = load_frag(reinterpret_cast<const E *>(
            stg + ST::at(mt * 16 + c16, (dc * 32 + g * 8) * (int)sizeof(E) / 16)));
    const bool need_mask = k0 + KT - 1 > p;
#pragma unroll
    for (int blk = 0; blk < BPT; ++blk) {
      float v[4 * MPB];
#pragma unroll
      for (int mm = 0; mm < MPB; ++mm) {
        const int mt = blk * MPB + mm;
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) c = mfma_chunk(cur[mt][dc], bq[dc], c);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[mm * 4 + i] = (need_mask && k0 + mt * 16 + g * 4 + i > p) ? -INFINITY : c[i];
      }
      const float mx = max_groups(max_chain<4 * MPB>(v));
      if (g == 0 && c16 < R) s_m[c16][tile * BPT + blk] = mx;
    }
  };
  // Key tiles are claimed at run time from the workgroup's counter (each wave's first is
  // its own index): with a fixed share per wave the waves of one compute unit finished
  // their streams up to a third of the kernel apart, the unit's loads in flight thinning
  // out as they did. A block's maximum does not depend on the wave that pools it.
  const int ntv = (int)min((long)NTW, (p - kb0) / KT + 1);  // tiles with a visible key
  auto claim = [&]() {
    int t = 0;
    if (lane == 0) t = atomicAdd(&s_next, 1);
    return __builtin_amdgcn_readfirstlane(t);
  };
  // double-buffered key tiles: the next tile's pieces load while this one computes. The
  // prefetches are unconditional too: a tile past the last re-reads the last one rather
  // than branch around the load. Claims only grow, so a wave stops at the first tile past
  // the range, and every tile claimed below it is pooled.
  u32x4 fa[ST::PPL], fb[ST::PPL];
  int ta = w, tb = claim();
  fetch(min(ta, ntv - 1), fa);
  while (ta < ntv) {
    fetch(min(tb, ntv - 1), fb);
    const int tc = claim();
    pool(ta, fa);
    if (tb >= ntv) break;
    fetch(min(tc, ntv - 1), fa);
    const int td = claim();
    pool(tb, fb);
    ta = tc;
    tb = td;
  }
  __syncthreads();

  const int m = a.top_k - 1;
  const int nv = max(0, min(SEL_NBLK, local - c0));  // candidates: blocks c0.. before `local`
  const int n_wg = gridDim.x;
  for (int r = w; r < R; r += SEL_WAVES) {  // one wave per group
    if (m == 0) break;
    uint32_t key[4];
    int32_t idx[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int cl = s4 * 64 + lane;
      idx[s4] = c0 + cl;
      key[s4] = cl < nv ? order_key(s_m[r][cl]) : 0u;
    }
    uint32_t ks = 0;
    int32_t is = 0x7fffffff;
    uint32_t *lk = reinterpret_cast<uint32_t *>(s_raw) + w * 2 * SELECT_LDS;
    if (nv > m) wave_threshold<4>(key, idx, m, lk, reinterpret_cast<int32_t *>(lk + SELECT_LDS), ks, is);
    uint32_t *ck = a.cand_key + (((long)b * R + r) * n_wg + wg) * m;
    int32_t *ci = a.cand_idx + (((long)b * R + r) * n_wg + wg) * m;
    int pos = 0;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const bool pr = taken(key[s4], idx[s4], ks, is);
      const uint64_t mk = ballot(pr);
      if (pr) {
        ck[pos + rank_below(mk)] = key[s4];
        ci[pos + rank_below(mk)] = idx[s4];
      }
      pos += popc64(mk);
    }
    if (lane >= pos && lane < m) {  // fewer than m candidates in this range
      ck[lane] = 0u;
      ci[lane] = -1;
    }
  }
}

template <typename E, int DI, int BS>
hipError_t launch_select_t(const IndexArgs &a, hipStream_t s) {
  const long blocks = a.q_start / BS + 1;  // blocks 0 .. local
  dim3 grid((unsigned)((blocks + SEL_NBLK - 1) / SEL_NBLK), 1, (unsigned)a.batch);
  hipLaunchKernelGGL((index_select_decode<E, DI, BS>), grid, dim3(SEL_WAVES * 64), 0, s, a);
  return hipGetLastError();
}

template <typename E, int DI, int BS>
hipError_t launch_prefill_t(const IndexArgs &a, hipStream_t s) {
  const int TQ = WG_COLS / a.h_kv;
  const long keys = (long)a.q_start + a.n_q;  // last position + 1
  dim3 grid((unsigned)((a.n_q + TQ - 1) / TQ), (unsigned)((keys + a.key_chunk - 1) / a.key_chunk),
            (unsigned)a.batch);
  // the counted flush needs whole, aligned runs in every row and a spare destination
  const bool cf = a.spare && a.n_blocks % OUT_RUN == 0 && (a.key_chunk / BS) % OUT_RUN == 0;
  if (a.rkey && cf)
    hipLaunchKernelGGL((index_pool_prefill<E, DI, BS, true, true>), grid, dim3(256), 0, s, a);
  else if (a.rkey)
    hipLaunchKernelGGL((index_pool_prefill<E, DI, BS, true, false>), grid, dim3(256), 0, s, a);
  else if (cf)
    hipLaunchKernelGGL((index_pool_prefill<E, DI, BS, false, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((index_pool_prefill<E, DI, BS, false, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename E, int DI, int BS>
hipError_t launch_decode_t(const IndexArgs &a, hipStream_t s) {
  const long keys = (long)a.q_start + 1;
  dim3 grid((unsigned)((keys + a.key_chunk - 1) / a.key_chunk), 1, (unsigned)a.batch);
  hipLaunchKernelGGL((index_pool_decode<E, DI, BS>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename E>
hipError_t pick_select(const IndexArgs &a, int d_idx, int bs, hipStream_t s) {
#define MSA_CASE(DI, BS) \
  if (d_idx == DI && bs == BS) return launch_select_t<E, DI, BS>(a, s);
  MSA_CASE(32, 32)
  MSA_CASE(32, 64)
  MSA_CASE(64, 32)
  MSA_CASE(64, 64)
#undef MSA_CASE
  return hipErrorInvalidValue;
}

template <typename E>
hipError_t pick(const IndexArgs &a, int d_idx, int bs, bool decode, hipStream_t s) {
#define MSA_CASE(DI, BS)                                                             \
  if (d_idx == DI && bs == BS)                                                       \
    return decode ? launch_decode_t<E, DI, BS>(a, s) : launch_prefill_t<E, DI, BS>(a, s);
  MSA_CASE(32, 32)
  MSA_CASE(32, 64)
  MSA_CASE(64, 32)
  MSA_CASE(64, 64)
#undef MSA_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fill(float *p, size_t n, float value, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, value);
  return hipGetLastError();
}

hipError_t launch_index_prefill(const IndexArgs &a, int dtype, int d_idx, int block_size,
                                hipStream_t s) {
  return dtype == 0 ? pick<float>(a, d_idx, block_size, false, s)
                    : pick<bf16_t>(a, d_idx, block_size, false, s);
}

hipError_t launch_index_select_decode(const IndexArgs &a, int dtype, int d_idx, int block_size,
                                      hipStream_t s) {
  return dtype == 0 ? pick_select<float>(a, d_idx, block_size, s)
                    : pick_select<bf16_t>(a, d_idx, block_size, s);
}

hipError_t launch_index_decode(const IndexArgs &a, int dtype, int d_idx, int block_size,
                               hipStream_t s) {
  return dtype == 0 ? pick<float>(a, d_idx, block_size, true, s)
                    : pick<bf16_t>(a, d_idx, block_size, true, s);
}

}  // namespace msa
