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
//      largest of the 64 lane maxima, with its low 16 bits cleared (only the
//      high bits are searched), theta, bounds the answer from below: 15
//      lanes each own a candidate >= theta, so every one of the 15 best
//      candidates is >= theta.
//   2. Candidates >= theta (usually a few dozen) are compacted into LDS in
//      ascending block order; if more than 64 survive (massive ties), an
//      exact search over all candidates is used instead.
//   3. The exact 15th-largest key T among the survivors is found bit by bit
//      with wave ballots; every survivor above T is kept, and the lowest-index
//      survivors equal to T fill the remaining slots.
//   4. Kept blocks are written in ascending order, then the local block.
#include "msa_device.h"
#include "msa_kernels.h"
#include "topk_rows.h"

namespace msa {

struct TopkArgs {
  Problem p;
  const float* scores;  // row R = r * hkv + g at scores + (R - r_base) * ld
  int64_t ld;
  int32_t* sel;
  int hkv_shift;
  int64_t r_base;       // first (row, group) index of the batch: cu_q[0] * hkv
};

__global__ __launch_bounds__(256) void block_topk_kernel(TopkArgs a) {
  __shared__ uint32_t surv_key[4][64];
  __shared__ int32_t surv_idx[4][64];
  const Problem& p = a.p;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // row values stay scalar
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
  // Registers sized to the row: a short row loads, keys and compacts only the
  // groups of 64 candidates it has.
  if (c <= 2 * 64)
    select_row<true, true, 2>(row, c, out, surv_key[wave], surv_idx[wave]);
  else if (c <= 4 * 64)
    select_row<true, true, 4>(row, c, out, surv_key[wave], surv_idx[wave]);
  else if (c <= 8 * 64)
    select_row<true, true, 8>(row, c, out, surv_key[wave], surv_idx[wave]);
  else if (c <= 12 * 64)
    select_row<true, true, 12>(row, c, out, surv_key[wave], surv_idx[wave]);
  else if (c <= kCached * 64)
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
  __shared__ uint32_t cand_key[kSplitWaves][kKeep];
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
  split_select_row<kSplitWaves>(a.scores + (R - a.r_base) * a.ld, c, out, surv_key, surv_idx, cand, cand_key);
  if (wave == 0 && lane == 0) out[kKeep] = c;
}

// Many long rows (a prefill chunk over a long cache): one workgroup of 4
// waves per row, each wave holding its quarter of the row (up to 36
// candidates per lane, rows of up to 9216 blocks) in registers, so the row is
// read from memory once; the one-wave kernel would read rows longer than
// 1024 blocks twice.  Same selection rule as the split kernel.
constexpr int kRowWaves = 4;
constexpr int kRowCached = 36;

__global__ __launch_bounds__(kRowWaves * 64) void block_topk_row4_kernel(TopkArgs a) {
  __shared__ uint32_t surv_key[kRowWaves][64];
  __shared__ int32_t surv_idx[kRowWaves][64];
  __shared__ int32_t cand[kRowWaves][kKeep];
  __shared__ uint32_t cand_key[kRowWaves][kKeep];
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
  split_select_row<kRowWaves, kRowCached>(a.scores + (R - a.r_base) * a.ld, c, out, surv_key, surv_idx, cand,
                                          cand_key);
  if (wave == 0 && lane == 0) out[kKeep] = c;
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
  if (max_blocks > (int64_t)kCached * 64) {
    hipLaunchKernelGGL(block_topk_row4_kernel, dim3((unsigned)rows), dim3(kRowWaves * 64), 0, stream, a);
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
