// msa_kernels.h — internal interface between the C-ABI host layer
// (msa_api.hip) and the kernel files.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace msa {

// Everything a kernel needs about the batch and the cache, by value.
struct Problem {
  // geometry
  int hq, hkv, head_dim, index_dim, group;  // group = hq / hkv
  float scale_log2e;                         // softmax scale * log2(e)
  // batch
  int num_seqs, total_q;
  int max_q_per_seq;        // max over sequences of their query rows (host mirror)
  const int32_t* seq_lens;  // device
  const int32_t* cu_q;      // device
  // cache
  const uint16_t* k;        // bf16 [num_blocks][128][hkv][head_dim]
  const uint16_t* v;
  const uint16_t* k_idx;    // bf16 [num_blocks][128][index_dim]
  const int32_t* block_table;
  int num_blocks, max_blocks_per_seq;
};

hipError_t launch_kv_append(const Problem& p, uint16_t* k_cache, uint16_t* v_cache, uint16_t* k_idx_cache,
                            const uint16_t* k_new, const uint16_t* v_new, const uint16_t* k_idx_new,
                            int max_q_per_seq, hipStream_t stream);

// first_row: the batch's first query row (cu_q[0]); scores holds that row first.
hipError_t launch_index_score(const Problem& p, const uint16_t* q_idx, float* scores, int64_t ld,
                              const int32_t* seq_lens_host, const int32_t* cu_q_host, hipStream_t stream,
                              int64_t first_row = 0);

// Selection quality (sampled rows): per-block attention mass over every
// causal token (sel NULL) or over the selected blocks' tokens, and coverage,
// recall and the indexer KL.
hipError_t launch_block_attn_mass(const Problem& p, const uint16_t* q, const int32_t* sel, const int32_t* rows,
                                  int32_t n_rows, float* mass, int64_t ld, hipStream_t stream);
hipError_t launch_selection_quality(const Problem& p, const int32_t* rows, int32_t n_rows, const float* mass,
                                    const float* sel_mass, const float* scores, const int32_t* sel, int64_t ld,
                                    float* quality, hipStream_t stream);
// max_blocks: blocks of the longest sequence (host-side), picks the kernel.
// first_row: the batch's first query row (cu_q[0]); sel is addressed by the
// batch's row numbers, scores from first_row on (its row 0 is row first_row).
hipError_t launch_block_topk(const Problem& p, const float* scores, int64_t ld, int32_t* sel, int64_t max_blocks,
                             hipStream_t stream, int64_t first_row = 0);

// Writes {seq_len, row_begin, row_end} to meta: the device arrays of a
// one-sequence sub-batch (seq_lens = meta, cu_q = meta + 1).
hipError_t launch_write_subbatch(int32_t* meta, int32_t seq_len, int32_t row_begin, int32_t row_end,
                                 hipStream_t stream);

// Largest max_blocks_per_seq the prefill selection inversion supports (its
// per-workgroup LDS histogram holds one counter per logical block).
constexpr int kMaxPrefillBlocks = 16384;

// Prefill Main Branch (blocks outer, queries inner) and its workspace: the
// plan (selection inversion) followed by the partial outputs.  The one-call
// form plans into the start of `ws` and runs with the partials after it.
size_t prefill_workspace_bytes(const Problem& p);
size_t prefill_plan_bytes(const Problem& p);
size_t prefill_run_bytes(const Problem& p);
hipError_t launch_attn_prefill(const Problem& p, const uint16_t* q, const int32_t* sel, uint16_t* out, void* ws,
                               hipStream_t stream);
hipError_t launch_attn_prefill_plan(const Problem& p, const int32_t* sel, void* plan, hipStream_t stream);
hipError_t launch_attn_prefill_run(const Problem& p, const uint16_t* q, const int32_t* sel, const void* plan,
                                   uint16_t* out, void* part, hipStream_t stream);

// Decode Main Branch (one query per sequence, split over its selected blocks).
size_t decode_workspace_bytes(const Problem& p);
hipError_t launch_attn_decode(const Problem& p, const uint16_t* q, const int32_t* sel, uint16_t* out, void* ws,
                              hipStream_t stream);
// The fused decode step (one query row per sequence): the append of each
// sequence's new token fused into the K_idx scan (which also clears the
// attention kernel's counters), then, for batches of fewer than 128
// (sequence, group) pairs, the selection, the attention and the merge in one
// kernel (larger batches: the top-k kernel, then the one-workgroup-per-pair
// attention).  Results equal msa_kv_append, msa_index_score, msa_block_topk
// and msa_sparse_attn_decode in sequence, bit for bit.  max_blocks: blocks of
// the longest sequence (host-side).
size_t decode_step_workspace_bytes(const Problem& p);
int32_t* decode_step_counters(const Problem& p, void* ws);  // NULL when the batch needs none
hipError_t launch_decode_append_score(const Problem& p, uint16_t* k_cache, uint16_t* v_cache, uint16_t* k_idx_cache,
                                      const uint16_t* k_new, const uint16_t* v_new, const uint16_t* k_idx_new,
                                      const uint16_t* q_idx, float* scores, int64_t ld, int32_t* counters,
                                      const int32_t* seq_lens_host, const int32_t* cu_q_host, hipStream_t stream);
hipError_t launch_decode_step_attn(const Problem& p, const uint16_t* q, const float* scores, int64_t ld, int32_t* sel,
                                   uint16_t* out, void* ws, int64_t max_blocks, hipStream_t stream);
// The library's static decode scratch (for callers that cannot allocate): the
// bytes this batch needs of it (0 when the one-workgroup-per-pair kernel runs),
// its capacity, and its device address on `device` (looked up once per device).
size_t decode_scratch_need(const Problem& p);
size_t decode_scratch_capacity();
hipError_t decode_scratch(int device, void** addr);

// Dense causal attention over the same cache (queries outer, no workspace).
hipError_t launch_dense_prefill(const Problem& p, const uint16_t* q, uint16_t* out, hipStream_t stream);

// Dense decode (one query per sequence, context split over workgroups and
// merged); max_ctx_blocks: blocks of the longest context (host-side).
size_t dense_decode_workspace_bytes(const Problem& p, int max_ctx_blocks);
hipError_t launch_dense_decode(const Problem& p, const uint16_t* q, uint16_t* out, void* ws, int max_ctx_blocks,
                               hipStream_t stream);

}  // namespace msa
