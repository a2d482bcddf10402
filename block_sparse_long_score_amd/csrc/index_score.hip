// index_score.hip — Index Branch scoring fused with the 128-token block
// max-pool.
//
// Source: "MiniMax 模型迭代与竞品分析：从 Text-01、M1、M2 到 M3", §2, MSA
// inference steps 1-2: per GQA group a light Q_idx scores the whole causal
// context against one K_idx per token shared by all groups; the token scores
// of each 128-token block are reduced by max so that a single strong token
// lets its block be recalled.  "MiniMax：Text-01 / M1 → M2.7 → M3", §5: the
// Index Branch works per GQA group.
//
// Mapping onto gfx950.  The scores of one tile form the product
//     S^T[keys x columns] = K_idx[keys x d_idx] * Q_idx^T[d_idx x columns],
// where a column is one (query, group) pair: the columns of consecutive query
// rows are consecutive rows of the flattened Q_idx [total_q*Hkv][d_idx], so a
// 32-column MFMA tile is 32/Hkv queries times all Hkv groups, and one K_idx
// tile serves every group.  Keys sit on the MFMA M axis, so the 32x32 output
// leaves 16 keys of one column in each lane's accumulators: the block max is
// an in-lane max over the 4 key tiles of a block plus one exchange between the
// two wave halves.  Token scores never leave registers; only one fp32 value
// per (query, group, block) is written, staged through LDS so that each
// (query, group) row is written as one contiguous run.
//
// Work split.  A workgroup (4 waves) owns a tile of 32*NCT columns (queries
// aligned to absolute positions, so the tile lies inside one 128-token block)
// and a chunk of `kc` key blocks; wave w takes blocks w, w+4, ... of the chunk.
// Every wave keeps the whole Q_idx tile in registers and streams K_idx from
// the cache through the block table.  Only the query tile's own block needs a
// causal mask (key position > query position).
#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {

struct IndexArgs {
  Problem p;
  const uint16_t* q_idx;
  float* out;
  int64_t ld;
  int tq;         // queries per tile = 32 * NCT / hkv
  int hkv_shift;  // log2(hkv)
  int kc;         // key blocks per workgroup
  int64_t first_row;  // out holds rows [first_row, first_row + total_q) of the batch, from its start
};

// Pooled scores of one key block for every column tile, returned per lane
// (lanes l and l^32 hold the two halves of column l%32 before the exchange).
// DIAG: the block holds the query tile itself; keys after a column's query
// position are masked.
template <int DIDX, int NCT, bool DIAG>
__device__ __forceinline__ void pool_block(const uint16_t* __restrict__ kbase, const bf16x8 (&bq)[NCT][DIDX / 16],
                                           const int (&lim)[NCT], float (&runmax)[NCT]) {
  constexpr int KS = DIDX / 16;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) runmax[ct] = -__builtin_inff();
  // One 32-key tile at a time, the next tile's K_idx loaded while this one is
  // multiplied: KS 16-byte loads per lane per tile.
  bf16x8 ak[KS], ak_next[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) ak[ks] = as_bf16x8(load16(kbase + l32 * DIDX + ks * 16));
  // The masked (diagonal) block keeps the key-tile loop rolled so its
  // per-element masks are formed inside the loop instead of all up front.
  constexpr int kUnroll = DIAG ? 1 : 4;
#pragma unroll kUnroll
  for (int m = 0; m < 4; ++m) {
    __builtin_amdgcn_sched_barrier(0);
    if (m < 3) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ak_next[ks] = as_bf16x8(load16(kbase + ((m + 1) * 32 + l32) * DIDX + ks * 16));
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x16 acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma32(ak[ks], bq[ct][ks], acc);
      if constexpr (DIAG) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = m * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          acc[r] = key > lim[ct] ? -__builtin_inff() : acc[r];
        }
      }
      float mx = acc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, acc[r]);
      runmax[ct] = fmaxf(runmax[ct], mx);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ak[ks] = ak_next[ks];
  }
}

template <int DIDX, int NCT>
__global__ __launch_bounds__(256, 2) void index_score_kernel(IndexArgs a) {
  constexpr int KS = DIDX / 16;  // MFMA k-steps over the index dimension
  constexpr int NC = 32 * NCT;   // columns per workgroup
  extern __shared__ float pooled_s[];  // [NC][kc + 1]
  const Problem& p = a.p;

  const int s = blockIdx.z;
  const int row0 = p.cu_q[s];
  const int nq = p.cu_q[s + 1] - row0;
  if (nq <= 0) return;
  const int seq_len = p.seq_lens[s];
  const int first_pos = seq_len - nq;
  const int tq = a.tq;
  const int tile0 = (first_pos / tq) * tq;
  const int n_tiles = (seq_len - 1 - tile0) / tq + 1;
  if ((int)blockIdx.x >= n_tiles) return;
  const int p0 = tile0 + (n_tiles - 1 - (int)blockIdx.x) * tq;  // late (heavy) tiles first
  const int c_tile = p0 >> 7;
  const int kb0 = blockIdx.y * a.kc;
  if (kb0 > c_tile) return;
  const int nkb = min(a.kc, c_tile + 1 - kb0);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int ld_s = a.kc + 1;
  const int hkv_mask = (1 << a.hkv_shift) - 1;

  // This lane's column in every column tile, and its Q_idx operand.
  bf16x8 bq[NCT][KS];
  int col_pos[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int col = ct * 32 + l32;
    const int pos = p0 + (col >> a.hkv_shift);
    const bool valid = pos >= first_pos && pos < seq_len;
    col_pos[ct] = pos;
    const int64_t R = ((int64_t)(row0 + pos - first_pos) << a.hkv_shift) + (col & hkv_mask);
    const uint16_t* src = a.q_idx + R * DIDX + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = valid ? load16(src + ks * 16) : u32x4{0u, 0u, 0u, 0u};
      bq[ct][ks] = as_bf16x8(v);
    }
  }

  const int32_t* table = p.block_table + (int64_t)s * p.max_blocks_per_seq;
  const int tab = lane < nkb ? table[kb0 + lane] : -1;  // the chunk's table entries, one per lane (kc <= 64)
  for (int kb = kb0 + wave; kb < kb0 + nkb; kb += 4) {
    const int phys = __builtin_amdgcn_readlane(tab, kb - kb0);
    float runmax[NCT];
    if (phys >= 0 && phys < p.num_blocks) {
      const uint16_t* kbase = p.k_idx + (int64_t)phys * kBlock * DIDX + half * 8;
      if (kb == c_tile) {
        int lim[NCT];  // in-block index of each column's query: later keys are masked
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) lim[ct] = col_pos[ct] - kb * kBlock;
        pool_block<DIDX, NCT, true>(kbase, bq, lim, runmax);
      } else {
        const int lim[NCT] = {};
        pool_block<DIDX, NCT, false>(kbase, bq, lim, runmax);
      }
    } else {
      // A block the table does not map holds no keys: the max over no scores.
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) runmax[ct] = -__builtin_inff();
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float v = fmaxf(runmax[ct], swap_halves(runmax[ct]));
      if (half == 0) pooled_s[(ct * 32 + l32) * ld_s + (kb - kb0)] = v;
    }
  }
  __syncthreads();

  // Each valid (query, group) row writes its nkb pooled scores contiguously.
  for (int idx = threadIdx.x; idx < NC * nkb; idx += blockDim.x) {
    const int col = idx / nkb;
    const int j = idx - col * nkb;
    const int pos = p0 + (col >> a.hkv_shift);
    if (pos < first_pos || pos >= seq_len) continue;
    const int64_t R = ((int64_t)(row0 + pos - first_pos) << a.hkv_shift) + (col & hkv_mask);
    float v = pooled_s[col * ld_s + j];
    v = (v == 0.0f) ? 0.0f : v;  // -0 and +0 are the same score
    a.out[(R - (a.first_row << a.hkv_shift)) * a.ld + kb0 + j] = v;
  }
}

// Prefill variant: the WAVES waves of a workgroup share each K_idx block
// through LDS (double-buffered, filled by direct global-to-LDS loads) and
// each owns its own 32*NCTW columns, so a block fetched once feeds
// WAVES*32*NCTW columns (512 at 8 waves x 64 columns: 64 queries x 8 groups).
// Eight waves of <= 128 VGPRs give four waves per SIMD to interleave the
// MFMA stream with the max reductions.  Blocks at or after the tile's first
// query block are masked per column (key position > query position).  Pooled
// scores are staged in LDS and written as one contiguous run per (query,
// group) row.
constexpr int kSharedFlush = 16;  // pooled scores staged in LDS per flush

// LDS layout of a staged K_idx block: rows of DIDX bf16 without padding, the
// 16-byte chunk c of row r stored at chunk position c ^ swz(r), where swz
// spreads the 16 rows one MFMA operand read touches over distinct banks
// (rows per 256 bytes: 2 at DIDX=64, 4 at DIDX=32).
template <int DIDX>
__device__ __forceinline__ int kidx_swizzle(int r, int c) {
  constexpr int CPR = DIDX / 8;          // 16-byte chunks per row
  constexpr int RPB = 256 / (DIDX * 2);  // rows per 256 bytes of banks
  return c ^ ((r / RPB) & (CPR - 1));
}

// Pooled scores of one LDS-staged key block for a wave's 16-column tiles,
// on the 16x16x32 bf16 MFMA with keys on M: A lane l holds K_idx[key l%16]
// [8*(l/16) .. +7] of a 32-wide k-step, B lane l holds Q_idx[column l%16]
// likewise, and D lane l register i holds the score of key 4*(l/16)+i for
// column l%16.  The 8 key tiles of the block are software-pipelined over two
// accumulator sets, so each tile's running max overlaps the next tile's
// MFMAs.  Each lane keeps a running max over its 4-key subsets; the four
// lanes of a column are combined by the caller.  MASKED: keys after a
// column's query position are -inf.
template <int DIDX, int NCT, bool MASKED>
__device__ __forceinline__ void shared_pool(const uint16_t* __restrict__ kt, const bf16x8 (&bq)[NCT][DIDX / 32],
                                            const int (&lim)[NCT], float (&runmax)[NCT]) {
  constexpr int KS = DIDX / 32;
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, q4 = lane >> 4;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) runmax[ct] = -__builtin_inff();
  f32x4 acc[2][NCT];
  auto issue = [&](int t, f32x4 (&a)[NCT]) {
    bf16x8 ak[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int r = t * 16 + l16;
      ak[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(&kt[r * DIDX + kidx_swizzle<DIDX>(r, ks * 4 + q4) * 8]));
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      a[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) a[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[ks], bq[ct][ks], a[ct], 0, 0, 0);
    }
  };
  auto reduce = [&](int t, f32x4 (&a)[NCT]) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 v = a[ct];
      if constexpr (MASKED) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = t * 16 + 4 * q4 + i > lim[ct] ? -__builtin_inff() : v[i];
      }
      runmax[ct] = fmaxf(fmaxf(fmaxf(fmaxf(runmax[ct], v[0]), v[1]), v[2]), v[3]);  // two v_max3
    }
  };
  issue(0, acc[0]);
#pragma unroll
  for (int t = 1; t < kBlock / 16; ++t) {
    issue(t, acc[t & 1]);
    reduce(t - 1, acc[(t - 1) & 1]);
  }
  reduce(kBlock / 16 - 1, acc[1]);
}

// Monotone map float -> uint32 (a < b as numbers <=> key(a) < key(b), with
// -0 just below +0) and its inverse.
__device__ __forceinline__ uint32_t pool_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// The largest of the four lanes that share a column (lanes l%16 + 16j), on
// pool keys: each swap leaves a lane's own value and its partner's in the two
// results, so one integer max combines them, with no select and no float
// canonicalisation.
__device__ __forceinline__ uint32_t column_max_key16(uint32_t k) {
  const auto a = __builtin_amdgcn_permlane32_swap(k, k, false, false);
  k = max(a[0], a[1]);  // lanes l and l ^ 32
  const auto b = __builtin_amdgcn_permlane16_swap(k, k, false, false);
  return max(b[0], b[1]);  // and l ^ 16
}

template <int DIDX, int NCTW, int WAVES>
__global__ __launch_bounds__(64 * WAVES, WAVES / 2) void index_score_shared_kernel(IndexArgs a) {
  constexpr int KS = DIDX / 32;           // 16x16x32 MFMA k-steps
  constexpr int NCT = 2 * NCTW;           // 16-column tiles per wave
  constexpr int NCW = 32 * NCTW;          // columns per wave
  constexpr int NC = WAVES * NCW;         // columns per workgroup
  constexpr int BLK = kBlock * DIDX;      // bf16 elements of one K_idx block
  __shared__ __attribute__((aligned(1024))) uint16_t kbuf[2][BLK];
  __shared__ uint32_t pooled_s[NC][kSharedFlush + 1];  // pool keys of the pooled scores
  __shared__ int32_t tab_s[64];
  __shared__ int64_t colrow_s[NC];  // each column's row of pooled scores (offset into a.out)
  __shared__ int32_t colpos_s[NC];  // each column's query position (-1: no query in this column)
  const Problem& p = a.p;

  const int s = blockIdx.z;
  const int row0 = p.cu_q[s];
  const int nq = p.cu_q[s + 1] - row0;
  if (nq <= 0) return;
  const int seq_len = p.seq_lens[s];
  const int first_pos = seq_len - nq;
  const int tq = a.tq;  // = NC / hkv
  const int tile0 = (first_pos / tq) * tq;
  const int n_tiles = (seq_len - 1 - tile0) / tq + 1;
  if ((int)blockIdx.x >= n_tiles) return;
  const int p0 = tile0 + (n_tiles - 1 - (int)blockIdx.x) * tq;  // late (heavy) tiles first
  const int plo = max(p0, first_pos);
  const int phi = min(p0 + tq, seq_len) - 1;
  const int c_hi = phi >> 7;   // last block any column needs
  const int kb0 = blockIdx.y * a.kc;
  if (kb0 > c_hi) return;
  const int nkb = min(a.kc, c_hi + 1 - kb0);
  const int unmasked_end = (plo + 1) >> 7;  // blocks below this are fully causal for every column

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, q4 = lane >> 4;
  const int hkv_mask = (1 << a.hkv_shift) - 1;

  // This lane's column in every 16-column tile and its Q_idx operand
  // (dims 32*ks + 8*q4 .. +7).
  bf16x8 bq[NCT][KS];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int col = wave * NCW + ct * 16 + l16;
    const int pos = p0 + (col >> a.hkv_shift);
    const bool valid = pos >= first_pos && pos < seq_len;
    const int64_t R = ((int64_t)(row0 + pos - first_pos) << a.hkv_shift) + (col & hkv_mask);
    const uint16_t* src = a.q_idx + R * DIDX + q4 * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bq[ct][ks] = as_bf16x8(valid ? load16(src + ks * 32) : u32x4{0u, 0u, 0u, 0u});
  }

  // Staging: direct global-to-LDS loads (16 bytes per lane, one contiguous
  // 1 KB LDS run per wave instruction).  Lane L of the instruction that fills
  // rows [8j, 8j+8) (DIDX=64) lands at chunk position L % CPR of row
  // 8j + L / CPR, so it loads the global chunk that the swizzle puts there.
  constexpr int CPR = DIDX / 8;                // 16-byte chunks per row
  constexpr int RUNS = BLK * 2 / 1024;         // 1 KB runs per block
  static_assert(RUNS % WAVES == 0, "runs per wave");
  // The chunk's block-table entries (kc <= 64) are staged in LDS once, so
  // each block's copy is requested without a dependent global load.
  const int32_t* table = p.block_table + (int64_t)s * p.max_blocks_per_seq;
  if (wave == 0) tab_s[lane] = lane < nkb ? table[kb0 + lane] : -1;
  for (int col = threadIdx.x; col < NC; col += blockDim.x) {
    const int pos = p0 + (col >> a.hkv_shift);
    const bool ok = pos >= first_pos && pos < seq_len;
    const int64_t R = ((int64_t)(row0 + pos - first_pos) << a.hkv_shift) + (col & hkv_mask);
    colrow_s[col] = ok ? (R - (a.first_row << a.hkv_shift)) * a.ld : 0;
    colpos_s[col] = ok ? pos : -1;
  }
  __syncthreads();
  auto dma = [&](int kb, int buf) {
    const int phys = tab_s[kb - kb0];
    const uint16_t* src = p.k_idx + (int64_t)((phys >= 0 && phys < p.num_blocks) ? phys : 0) * BLK;
#pragma unroll
    for (int k = 0; k < RUNS / WAVES; ++k) {
      const int run = wave + WAVES * k;
      const int row = run * (1024 / (DIDX * 2)) + lane / CPR;
      const int chunk = kidx_swizzle<DIDX>(row, lane % CPR);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + row * DIDX + chunk * 8),
                                       reinterpret_cast<__attribute__((address_space(3))) void*>(
                                           reinterpret_cast<uintptr_t>(&kbuf[buf][run * 512])),
                                       16, 0, 0);
    }
  };
  dma(kb0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Each valid (query, group) row writes the staged pooled scores of blocks
  // [kf, kf + n) it can see (b <= its own block) as one contiguous run.
  auto store = [&](int col, int kf, int j) {
    if (kf + j > (colpos_s[col] >> 7)) return;  // no query in the column, or a block after its own
    float v = key_to_float(pooled_s[col][j]);
    v = (v == 0.0f) ? 0.0f : v;  // -0 and +0 are the same score
    a.out[colrow_s[col] + kf + j] = v;
  };
  auto flush = [&](int kf, int n) {
    constexpr int kThreads = 64 * WAVES;
    // The thread index passes through an empty asm so the compiler derives
    // the flush's addresses here rather than holding them (in registers it
    // would spill) across the whole key-block loop.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    if (n == kSharedFlush) {  // a full flush: each thread keeps one block slot, columns step by kThreads / n
      const int j = tid % kSharedFlush;
      for (int col = tid / kSharedFlush; col < NC; col += kThreads / kSharedFlush) store(col, kf, j);
    } else {
      for (int idx = tid; idx < NC * n; idx += kThreads) store(idx / n, kf, idx % n);
    }
  };

  for (int i = 0; i < nkb; ++i) {
    const int kb = kb0 + i;
    if (i + 1 < nkb) dma(kb + 1, (i + 1) & 1);  // that buffer was released by the last barrier
    const uint16_t* kt = kbuf[i & 1];
    float runmax[NCT];
    if (kb >= unmasked_end) {
      int lim[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) lim[ct] = colpos_s[wave * NCW + ct * 16 + l16] - kb * kBlock;
      shared_pool<DIDX, NCT, true>(kt, bq, lim, runmax);
    } else {
      const int lim[NCT] = {};
      shared_pool<DIDX, NCT, false>(kt, bq, lim, runmax);
    }
    const int phys = tab_s[kb - kb0];
    if (!(phys >= 0 && phys < p.num_blocks)) {  // an unmapped block holds no keys (its copy read block 0)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) runmax[ct] = -__builtin_inff();
    }
    const int slot = i % kSharedFlush;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const uint32_t k = column_max_key16(pool_key(runmax[ct]));
      if (q4 == 0) pooled_s[wave * NCW + ct * 16 + l16][slot] = k;
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the next block have landed
    __syncthreads();
    if (slot == kSharedFlush - 1 || i + 1 == nkb) {
      flush(kb - slot, slot + 1);
      __syncthreads();
    }
  }
}

// Decode-shaped batches (one 32-column tile per sequence): each wave streams
// its own key blocks.  A block arrives by direct non-temporal global-to-LDS
// loads into the wave's own 16 KB LDS region (coalesced 1 KB runs, swizzled
// as in the prefill kernel), is read into registers, and the wave's next block is
// requested into the same region before this one is multiplied, so one block
// per wave is always in flight without a workgroup barrier.
// The fused decode step's append (APPEND): each sequence's new token (its
// single query row) is written into the cache by the workgroup that scores
// the token's block, before any of its waves copies that block, and that
// workgroup clears the sequence's rows of the attention kernel's counters.
struct StepAppend {
  uint16_t* k_cache;
  uint16_t* v_cache;
  uint16_t* k_idx_cache;
  const uint16_t* k_new;      // bf16 [total_q][hkv][D]
  const uint16_t* v_new;
  const uint16_t* k_idx_new;  // bf16 [total_q][d_idx]
  int32_t* counters;          // [total_q][hkv] or NULL
};

template <int DIDX, bool APPEND>
__global__ __launch_bounds__(256, 2) void index_score_stream_kernel(IndexArgs a, StepAppend ap) {
  constexpr int KS = DIDX / 16;          // 32x32x16 MFMA k-steps
  constexpr int BLK = kBlock * DIDX;     // bf16 elements of one K_idx block
  constexpr int CPR = DIDX / 8;          // 16-byte chunks per row
  constexpr int RUNS = BLK * 2 / 1024;   // 1 KB runs per block
  __shared__ __attribute__((aligned(1024))) uint16_t kbuf[4][BLK];
  extern __shared__ float pooled_s[];  // [32][kc + 1]
  const Problem& p = a.p;

  // APPEND: the grid is (tile, sequence, key chunk) with the chunks in reverse
  // order, so every sequence's last chunk (the one that appends the new
  // token before scoring it) is dispatched first and its extra work
  // overlaps the rest of the scan instead of lengthening its tail.
  const int s = APPEND ? blockIdx.y : blockIdx.z;
  const int key_chunk = APPEND ? (int)(gridDim.z - 1 - blockIdx.z) : (int)blockIdx.y;
  const int row0 = p.cu_q[s];
  const int nq = p.cu_q[s + 1] - row0;
  if (nq <= 0) return;
  const int seq_len = p.seq_lens[s];
  const int first_pos = seq_len - nq;
  const int tq = a.tq;
  const int tile0 = (first_pos / tq) * tq;
  const int n_tiles = (seq_len - 1 - tile0) / tq + 1;
  if ((int)blockIdx.x >= n_tiles) return;
  const int p0 = tile0 + (n_tiles - 1 - (int)blockIdx.x) * tq;
  const int c_tile = p0 >> 7;
  const int kb0 = key_chunk * a.kc;
  if (kb0 > c_tile) return;
  const int nkb = min(a.kc, c_tile + 1 - kb0);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int ld_s = a.kc + 1;
  const int hkv_mask = (1 << a.hkv_shift) - 1;

  bf16x8 bq[KS];
  const int col_pos = p0 + (l32 >> a.hkv_shift);
  {
    const bool valid = col_pos >= first_pos && col_pos < seq_len;
    const int64_t R = ((int64_t)(row0 + col_pos - first_pos) << a.hkv_shift) + (l32 & hkv_mask);
    const uint16_t* src = a.q_idx + R * DIDX + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bq[ks] = as_bf16x8(valid ? load16(src + ks * 16) : u32x4{0u, 0u, 0u, 0u});
  }

  const int32_t* table = p.block_table + (int64_t)s * p.max_blocks_per_seq;
  const int tab = lane < nkb ? table[kb0 + lane] : -1;  // the chunk's table entries, one per lane (kc <= 64)
  uint16_t* region = kbuf[wave];
  auto dma = [&](int kb) {
    const int phys = __builtin_amdgcn_readlane(tab, kb - kb0);
    const uint16_t* src = p.k_idx + (int64_t)((phys >= 0 && phys < p.num_blocks) ? phys : 0) * BLK;
#pragma unroll
    for (int run = 0; run < RUNS; ++run) {
      const int row = run * (1024 / (DIDX * 2)) + lane / CPR;
      const int chunk = kidx_swizzle<DIDX>(row, lane % CPR);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + row * DIDX + chunk * 8),
                                       reinterpret_cast<__attribute__((address_space(3))) void*>(
                                           reinterpret_cast<uintptr_t>(region + run * 512)),
                                       16, 0, kLoadNT);
    }
  };
  if constexpr (APPEND) {
    const int t_new = seq_len - 1;  // one query per sequence: the new token
    if ((t_new >> 7) >= kb0 && (t_new >> 7) < kb0 + nkb) {
      const int phys = table[t_new >> 7];
      if (phys >= 0 && phys < p.num_blocks) {  // (an unmapped block holds no keys, as in msa_kv_append)
        const int kv_vec = (p.hkv * p.head_dim) >> 3;  // 16-byte vectors of one token's K (and V)
        constexpr int ki_vec = DIDX >> 3;
        const int64_t slot = (int64_t)phys * kBlock + (t_new & 127);
        for (int v = threadIdx.x; v < 2 * kv_vec + ki_vec; v += blockDim.x) {
          if (v < kv_vec)
            store16(ap.k_cache + (slot * kv_vec + v) * 8, load16(ap.k_new + ((int64_t)row0 * kv_vec + v) * 8));
          else if (v < 2 * kv_vec)
            store16(ap.v_cache + (slot * kv_vec + v - kv_vec) * 8,
                    load16(ap.v_new + ((int64_t)row0 * kv_vec + v - kv_vec) * 8));
          else
            store16(ap.k_idx_cache + (slot * ki_vec + v - 2 * kv_vec) * 8,
                    load16(ap.k_idx_new + ((int64_t)row0 * ki_vec + v - 2 * kv_vec) * 8));
        }
      }
      if (ap.counters && (int)threadIdx.x < p.hkv) ap.counters[((int64_t)row0 << a.hkv_shift) + threadIdx.x] = 0;
      __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
      __syncthreads();                // and every wave's, before the block is copied
    }
  }
  int kb = kb0 + wave;
  if (kb < kb0 + nkb) dma(kb);
  for (; kb < kb0 + nkb; kb += 4) {
    __builtin_amdgcn_s_waitcnt(0);  // this block has landed in the region
    // Whole block into registers: key tile m, k-step ks -> 16 bytes per lane.
    bf16x8 ak[4][KS];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int r = m * 32 + l32;
        ak[m][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(&region[r * DIDX + kidx_swizzle<DIDX>(r, 2 * ks + half) * 8]));
      }
    __builtin_amdgcn_s_waitcnt(0);  // reads done before the region is refilled
    if (kb + 4 < kb0 + nkb) dma(kb + 4);
    const bool diag = kb == c_tile;  // the query's own block: keys after it are masked
    const int lim = col_pos - kb * kBlock;
    float runmax = -__builtin_inff();
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      f32x16 acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma32(ak[m][ks], bq[ks], acc);
      if (diag) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = m * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          acc[r] = key > lim ? -__builtin_inff() : acc[r];
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) runmax = fmaxf(runmax, acc[r]);
    }
    const int phys = __builtin_amdgcn_readlane(tab, kb - kb0);
    if (!(phys >= 0 && phys < p.num_blocks)) runmax = -__builtin_inff();  // an unmapped block holds no keys
    const float v = fmaxf(runmax, swap_halves(runmax));
    if (half == 0) pooled_s[l32 * ld_s + (kb - kb0)] = v;
  }
  __syncthreads();

  // Each valid (query, group) row writes its nkb pooled scores contiguously.
  for (int idx = threadIdx.x; idx < 32 * nkb; idx += blockDim.x) {
    const int col = idx / nkb;
    const int j = idx - col * nkb;
    const int pos = p0 + (col >> a.hkv_shift);
    if (pos < first_pos || pos >= seq_len) continue;
    const int64_t R = ((int64_t)(row0 + pos - first_pos) << a.hkv_shift) + (col & hkv_mask);
    float v = pooled_s[col * ld_s + j];
    v = (v == 0.0f) ? 0.0f : v;  // -0 and +0 are the same score
    a.out[(R - (a.first_row << a.hkv_shift)) * a.ld + kb0 + j] = v;
  }
}

template <int DIDX, int NCT>
static hipError_t launch_index_t(const IndexArgs& a, dim3 grid, hipStream_t stream) {
  const size_t lds = (size_t)32 * NCT * (a.kc + 1) * sizeof(float);
  hipLaunchKernelGGL((index_score_kernel<DIDX, NCT>), grid, dim3(256), lds, stream, a);
  return hipGetLastError();
}

static hipError_t launch_index_impl(const Problem& p, const uint16_t* q_idx, float* scores, int64_t ld,
                                    const int32_t* seq_lens_host, const int32_t* cu_q_host, hipStream_t stream,
                                    int64_t first_row, const StepAppend* append) {
  int hkv_shift = 0;
  while ((1 << hkv_shift) < p.hkv) ++hkv_shift;
  int max_q = 0;
  for (int s = 0; s < p.num_seqs; ++s) max_q = std::max(max_q, cu_q_host[s + 1] - cu_q_host[s]);
  if (max_q <= 0) return hipSuccess;
  // Prefill-shaped batches: 512 columns per workgroup sharing each K_idx block.
  constexpr int kSharedCols = 8 * 32 * 2;  // 8 waves x 64 columns
  if (max_q * p.hkv > 4 * kSharedCols) {
    if (append) return hipErrorInvalidValue;  // the append is fused only into the one-tile-per-sequence scan
    const int tq = kSharedCols / p.hkv;
    int max_tiles = 0, max_blocks = 0;
    for (int s = 0; s < p.num_seqs; ++s) {
      const int nq = cu_q_host[s + 1] - cu_q_host[s];
      if (nq <= 0) continue;
      const int L = seq_lens_host[s];
      const int t0 = ((L - nq) / tq) * tq;
      max_tiles = std::max(max_tiles, (L - 1 - t0) / tq + 1);
      max_blocks = std::max(max_blocks, (L - 1) / kBlock + 1);
    }
    // Key blocks per workgroup: each workgroup loads its 64 KB Q_idx tile
    // once, so longer chunks cut that traffic (at 1024 blocks, 32 instead of
    // 16 halves it and the pipelined 128K prefill step is ~3% faster); short
    // contexts keep 16 so the grid still fills the chip.
    // (kc <= 64 always: the kernels hold a chunk's block-table entries one per lane.)
    const int kc = max_blocks >= 1024 ? 64 : (max_blocks >= 512 ? 32 : 16);
    IndexArgs a{p, q_idx, scores, ld, tq, hkv_shift, kc, first_row};
    dim3 grid((unsigned)max_tiles, (unsigned)((max_blocks + kc - 1) / kc), (unsigned)p.num_seqs);
    if (p.index_dim == 64)
      hipLaunchKernelGGL((index_score_shared_kernel<64, 2, 8>), grid, dim3(512), 0, stream, a);
    else
      hipLaunchKernelGGL((index_score_shared_kernel<32, 2, 8>), grid, dim3(512), 0, stream, a);
    return hipGetLastError();
  }
  // Decode-shaped and small batches: each wave streams its own key blocks.
  const int nct = (max_q * p.hkv <= 32) ? 1 : 4;
  const int tq = 32 * nct / p.hkv;
  int max_tiles = 0, max_blocks = 0;
  int64_t work = 0;
  for (int s = 0; s < p.num_seqs; ++s) {
    const int nq = cu_q_host[s + 1] - cu_q_host[s];
    if (nq <= 0) continue;
    const int L = seq_lens_host[s];
    const int t0 = ((L - nq) / tq) * tq;
    const int tiles = (L - 1 - t0) / tq + 1;
    max_tiles = std::max(max_tiles, tiles);
    max_blocks = std::max(max_blocks, (L - 1) / kBlock + 1);
    work += (int64_t)tiles * ((t0 / kBlock + (L - 1) / kBlock) / 2 + 1);
  }
  // Decode tiles stream at least 2 blocks per wave so each wave's next block is in flight while it multiplies.
  // (At most 64 blocks per chunk: one block-table entry per lane.)
  int kc = (int)std::min<int64_t>(64, std::max<int64_t>(nct == 1 ? 8 : 4, (work / 8192 + 3) / 4 * 4));
  IndexArgs a{p, q_idx, scores, ld, tq, hkv_shift, kc, first_row};
  dim3 grid((unsigned)max_tiles, (unsigned)((max_blocks + kc - 1) / kc), (unsigned)p.num_seqs);
  if (nct == 1) {
    const size_t lds = (size_t)32 * (a.kc + 1) * sizeof(float);
    if (append) {
      const dim3 agrid(grid.x, grid.z, grid.y);  // (tile, sequence, chunk): see the kernel
      if (p.index_dim == 64)
        hipLaunchKernelGGL((index_score_stream_kernel<64, true>), agrid, dim3(256), lds, stream, a, *append);
      else
        hipLaunchKernelGGL((index_score_stream_kernel<32, true>), agrid, dim3(256), lds, stream, a, *append);
      return hipGetLastError();
    }
    const StepAppend none{};
    if (p.index_dim == 64)
      hipLaunchKernelGGL((index_score_stream_kernel<64, false>), grid, dim3(256), lds, stream, a, none);
    else
      hipLaunchKernelGGL((index_score_stream_kernel<32, false>), grid, dim3(256), lds, stream, a, none);
    return hipGetLastError();
  }
  if (append) return hipErrorInvalidValue;  // the append is fused only into the one-tile-per-sequence scan
  return p.index_dim == 64 ? launch_index_t<64, 4>(a, grid, stream) : launch_index_t<32, 4>(a, grid, stream);
}

hipError_t launch_index_score(const Problem& p, const uint16_t* q_idx, float* scores, int64_t ld,
                              const int32_t* seq_lens_host, const int32_t* cu_q_host, hipStream_t stream,
                              int64_t first_row) {
  return launch_index_impl(p, q_idx, scores, ld, seq_lens_host, cu_q_host, stream, first_row, nullptr);
}

hipError_t launch_decode_append_score(const Problem& p, uint16_t* k_cache, uint16_t* v_cache, uint16_t* k_idx_cache,
                                      const uint16_t* k_new, const uint16_t* v_new, const uint16_t* k_idx_new,
                                      const uint16_t* q_idx, float* scores, int64_t ld, int32_t* counters,
                                      const int32_t* seq_lens_host, const int32_t* cu_q_host, hipStream_t stream) {
  const StepAppend ap{k_cache, v_cache, k_idx_cache, k_new, v_new, k_idx_new, counters};
  return launch_index_impl(p, q_idx, scores, ld, seq_lens_host, cu_q_host, stream, 0, &ap);
}

}  // namespace msa
