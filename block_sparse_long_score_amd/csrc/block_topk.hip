// block_topk.hip — per (query, group) choice of the blocks the Main Branch
// attends to.
//
// Source: "MiniMax 模型迭代与竞品分析：从 Text-01、M1、M2 到 M3", §2, MSA
// inference step 3: 16 blocks per query and per GQA group, the local block
// counted as one of the 16 rather than added as a 17th.  "MiniMax：Text-01 /
// M1 → M2.7 → M3", §5 names an exp-free Top-k: the choice only compares block
// scores, so no softmax over them is ever formed.  Equal scores go to the
// lower block index.
//
// One wavefront per (query, group) row; candidates are the blocks b < c of
// the row (c = the local block).  Scores are compared through a monotone
// 32-bit key (order_key), which also makes -0 equal to +0.
//   1. Each lane takes the maximum key of its strided candidates; the 15th
//      largest of the 64 lane maxima, theta, bounds the answer from below:
//      the 15 lanes above it each own a candidate >= theta, so every one of
//      the 15 best candidates is >= theta.
//   2. Candidates >= theta (usually a few dozen) are compacted into LDS in
//      ascending block order; if more than 64 survive (massive ties), an
//      exact search over all candidates is used instead.
//   3. The exact 15th-largest key T among the survivors is found bit by bit
//      with wave ballots; every survivor above T is kept, and the lowest-index
//      survivors equal to T fill the remaining slots.
//   4. Kept blocks are written in ascending order, then the local block.
#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {

struct TopkArgs {
  Problem p;
  const float* scores;  // row R = r * hkv + g at scores + (R - r_base) * ld
  int64_t ld;
  int32_t* sel;
  int hkv_shift;
  int64_t r_base;       // first (row, group) index of the batch: cu_q[0] * hkv
};

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// k-th largest of the 64 lane values (k <= 64): the largest T with
// |{lanes : x >= T}| >= k, built from the top bit down.
__device__ __forceinline__ uint32_t kth_largest_lane(uint32_t x, int k) {
  uint32_t t = 0;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    if (__popcll(__ballot(x >= cand)) >= k) t = cand;
  }
  return t;
}

constexpr int kKeep = kTopK - 1;  // non-local blocks kept per row
constexpr int kCached = 16;       // candidates per lane held in registers (rows with c <= 1024)

// Keys of candidates j*64 + lane for j in [j0, j0 + kCached): one batch of
// independent loads (0 beyond the last candidate).
__device__ __forceinline__ void load_batch(const float* __restrict__ row, int c, int j0, uint32_t (&keys)[kCached]) {
  const int lane = threadIdx.x & 63;
  float v[kCached];
#pragma unroll
  for (int j = 0; j < kCached; ++j) {
    const int b = (j0 + j) * 64 + lane;
    v[j] = b < c ? row[b] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < kCached; ++j) keys[j] = (j0 + j) * 64 + lane < c ? order_key(v[j]) : 0u;
}

// Selection for one row.  Rows with c <= 1024 candidates keep their keys in
// registers; longer rows are streamed in batches of 1024 (16 per lane).
template <bool CACHED, bool WRITE_LOCAL = true>
__device__ void select_row(const float* __restrict__ row, int c, int32_t* __restrict__ out, uint32_t* surv_key,
                           int32_t* surv_idx) {
  const int lane = threadIdx.x & 63;
  const int nj = (c + 63) / 64;
  uint32_t keys[kCached];
  if constexpr (CACHED) load_batch(row, c, 0, keys);

  // 1. lane maxima and theta.
  uint32_t lmax = 0;
  for (int j0 = 0; j0 < nj; j0 += kCached) {
    if constexpr (!CACHED) load_batch(row, c, j0, keys);
#pragma unroll
    for (int j = 0; j < kCached; ++j) lmax = max(lmax, keys[j]);
  }
  const uint32_t theta = kth_largest_lane(lmax, kKeep);

  // 2. compact survivors (key >= theta) in ascending block order.
  int count = 0;
  for (int j0 = 0; j0 < nj; j0 += kCached) {
    if constexpr (!CACHED) load_batch(row, c, j0, keys);
#pragma unroll
    for (int j = 0; j < kCached; ++j) {
      const bool ok = keys[j] >= theta && keys[j] != 0u;
      const uint64_t m = __ballot(ok);
      const int pos = count + lanes_below(m);
      if (ok && pos < 64) {
        surv_key[pos] = keys[j];
        surv_idx[pos] = (j0 + j) * 64 + lane;
      }
      count += __popcll(m);
    }
  }
  wave_lds_sync();

  if (count <= 64) {
    // 3. exact threshold among the survivors.
    const bool have = lane < count;
    const uint32_t k = have ? surv_key[lane] : 0u;
    const int idx = have ? surv_idx[lane] : 0;
    const uint32_t T = kth_largest_lane(k, kKeep);
    const int need = kKeep - __popcll(__ballot(have && k > T));
    const uint64_t eq = __ballot(have && k == T);
    const bool take = have && (k > T || (k == T && lanes_below(eq) < need));
    const uint64_t tm = __ballot(take);
    // 4. ascending output, local block last.
    if (take) out[lanes_below(tm)] = idx;
  } else {
    // Massive ties: exact k-th largest over all candidates, bit by bit.
    auto key_at = [&](int j) -> uint32_t {
      const int b = j * 64 + lane;
      return b < c ? order_key(row[b]) : 0u;
    };
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      int n = 0;
      for (int j = 0; j < nj; ++j) n += __popcll(__ballot(key_at(j) >= cand));
      if (n >= kKeep) T = cand;
    }
    int gt = 0;
    for (int j = 0; j < nj; ++j) gt += __popcll(__ballot(key_at(j) > T));
    const int need = kKeep - gt;
    int taken = 0, ties = 0;
    for (int j = 0; j < nj && taken < kKeep; ++j) {
      const uint32_t k = key_at(j);
      const uint64_t eq = __ballot(k == T);
      const bool take = k > T || (k == T && ties + lanes_below(eq) < need);
      const uint64_t tm = __ballot(take);
      if (take) out[taken + lanes_below(tm)] = j * 64 + lane;
      taken += __popcll(tm);
      ties += __popcll(eq);
    }
  }
  if (WRITE_LOCAL && lane == 0) out[kKeep] = c;
}

__global__ __launch_bounds__(256) void block_topk_kernel(TopkArgs a) {
  __shared__ uint32_t surv_key[4][64];
  __shared__ int32_t surv_idx[4][64];
  const Problem& p = a.p;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t local = (int64_t)blockIdx.x * 4 + wave;
  if (local >= ((int64_t)p.total_q << a.hkv_shift)) return;
  const int64_t R = a.r_base + local;
  const int r = (int)(R >> a.hkv_shift);
  const int s = seq_of_row(p.cu_q, p.num_seqs, r);
  const int t = p.seq_lens[s] - (p.cu_q[s + 1] - r);
  const int c = t >> 7;
  int32_t* out = a.sel + R * kTopK;
  if (c + 1 <= kTopK) {
    if (lane < kTopK) out[lane] = lane <= c ? lane : -1;
    return;
  }
  const float* row = a.scores + (R - a.r_base) * a.ld;
  if (c <= kCached * 64)
    select_row<true>(row, c, out, surv_key[wave], surv_idx[wave]);
  else
    select_row<false>(row, c, out, surv_key[wave], surv_idx[wave]);
}

// Long rows when there are few of them (decode over very long contexts): one
// workgroup of kSplitWaves waves per row.  Wave w finds the exact top 15 of
// its contiguous share of the candidates (ties to the lower index, as above);
// the overall top 15 lies in the union of these, which wave 0 then searches
// in ascending block order with the same exact threshold and tie rule.
constexpr int kSplitWaves = 16;
constexpr int64_t kSplitMaxRows = 1024;    // split only while one wave per row leaves the chip idle
constexpr int64_t kSplitMinBlocks = 2048;  // and rows are long enough to be worth splitting

__global__ __launch_bounds__(kSplitWaves * 64) void block_topk_split_kernel(TopkArgs a) {
  __shared__ uint32_t surv_key[kSplitWaves][64];
  __shared__ int32_t surv_idx[kSplitWaves][64];
  __shared__ int32_t cand[kSplitWaves][kKeep];
  const Problem& p = a.p;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t R = a.r_base + blockIdx.x;
  const int r = (int)(R >> a.hkv_shift);
  const int s = seq_of_row(p.cu_q, p.num_seqs, r);
  const int t = p.seq_lens[s] - (p.cu_q[s + 1] - r);
  const int c = t >> 7;
  int32_t* out = a.sel + R * kTopK;
  if (c + 1 <= kTopK) {  // every causal block is kept
    if (wave == 0 && lane < kTopK) out[lane] = lane <= c ? lane : -1;
    return;
  }
  const float* row = a.scores + (R - a.r_base) * a.ld;
  // Shares are multiples of 64 candidates; a share of n <= 15 keeps all n.
  const int share = ((c + kSplitWaves * 64 - 1) / (kSplitWaves * 64)) * 64;
  const int lo = min(c, wave * share), n = min(share, c - lo);
  if (n > 0) {
    if (n <= kCached * 64)
      select_row<true, false>(row + lo, n, cand[wave], surv_key[wave], surv_idx[wave]);
    else
      select_row<false, false>(row + lo, n, cand[wave], surv_key[wave], surv_idx[wave]);
  }
  __syncthreads();
  if (wave != 0) return;
  // Candidates of all shares in ascending block order: up to kSplitWaves * 15.
  constexpr int kRounds = (kSplitWaves * kKeep + 63) / 64;
  uint32_t key[kRounds];
  int32_t idx[kRounds];
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const int e = j * 64 + lane;          // position in the concatenated list
    const int w = e / kKeep, k = e - w * kKeep;
    const int lo_w = min(c, w * share), n_w = min(share, c - lo_w);
    const bool have = w < kSplitWaves && k < min(n_w, kKeep);
    idx[j] = have ? lo_w + cand[w][k] : -1;
    key[j] = have ? order_key(row[idx[j]]) : 0u;
  }
  // Exact 15th-largest key over the candidates, bit by bit.
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cnd = T | (1u << bit);
    int nge = 0;
#pragma unroll
    for (int j = 0; j < kRounds; ++j) nge += __popcll(__ballot(key[j] >= cnd));
    if (nge >= kKeep) T = cnd;
  }
  int gt = 0;
#pragma unroll
  for (int j = 0; j < kRounds; ++j) gt += __popcll(__ballot(key[j] > T));
  const int need = kKeep - gt;
  int taken = 0, ties = 0;
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const uint64_t eq = __ballot(key[j] == T && idx[j] >= 0);
    const bool take = idx[j] >= 0 && (key[j] > T || (key[j] == T && ties + lanes_below(eq) < need));
    const uint64_t tm = __ballot(take);
    if (take) out[taken + lanes_below(tm)] = idx[j];
    taken += __popcll(tm);
    ties += __popcll(eq);
  }
  if (lane == 0) out[kKeep] = c;
}

hipError_t launch_block_topk(const Problem& p, const float* scores, int64_t ld, int32_t* sel, int64_t max_blocks,
                             hipStream_t stream, int64_t first_row) {
  int hkv_shift = 0;
  while ((1 << hkv_shift) < p.hkv) ++hkv_shift;
  const int64_t rows = (int64_t)p.total_q << hkv_shift;
  if (rows == 0) return hipSuccess;
  TopkArgs a{p, scores, ld, sel, hkv_shift, first_row << hkv_shift};
  if (rows <= kSplitMaxRows && max_blocks > kSplitMinBlocks) {
    hipLaunchKernelGGL(block_topk_split_kernel, dim3((unsigned)rows), dim3(kSplitWaves * 64), 0, stream, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(block_topk_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

__global__ void write_subbatch_kernel(int32_t* meta, int32_t seq_len, int32_t row_begin, int32_t row_end) {
  meta[0] = seq_len;
  meta[1] = row_begin;
  meta[2] = row_end;
}

hipError_t launch_write_subbatch(int32_t* meta, int32_t seq_len, int32_t row_begin, int32_t row_end,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(write_subbatch_kernel, dim3(1), dim3(1), 0, stream, meta, seq_len, row_begin, row_end);
  return hipGetLastError();
}

}  // namespace msa
