// msa_api.hip — the C ABI of libmsa (include/msa.h): host-side argument
// validation, then asynchronous kernel launches on the caller's stream.
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing and this file's checks can run on a machine without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "msa.h"
#include "msa_kernels.h"

namespace {

thread_local std::string g_last_error;

// msa_index_select: a 256-byte sub-batch descriptor, then the pooled scores
// of one chunk of query rows; the suggested size keeps them within ~192 MB,
// below the 256 MB Infinity Cache.
constexpr int64_t kSelectMetaBytes = 256;
constexpr int64_t kSelectScoresBudget = (int64_t)192 << 20;

msa_status fail(msa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

msa_status ok() {
  g_last_error.clear();
  return MSA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool pow2_upto32(int x) { return x >= 1 && x <= 32 && (x & (x - 1)) == 0; }

msa_status check_dims(const msa_dims* d) {
  if (!d) return fail(MSA_ERR_NULL_POINTER, "dims is NULL");
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0)
    return fail(MSA_ERR_BAD_SHAPE, "head counts must be positive (Hq=%d, Hkv=%d)", d->num_q_heads, d->num_kv_heads);
  if (d->num_q_heads % d->num_kv_heads != 0)
    return fail(MSA_ERR_BAD_SHAPE, "Hq=%d is not a multiple of Hkv=%d", d->num_q_heads, d->num_kv_heads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(MSA_ERR_UNSUPPORTED, "head_dim=%d (supported: 64, 128)", d->head_dim);
  if (d->index_dim != 32 && d->index_dim != 64)
    return fail(MSA_ERR_UNSUPPORTED, "index_dim=%d (supported: 32, 64)", d->index_dim);
  if (d->block_size != 128) return fail(MSA_ERR_UNSUPPORTED, "block_size=%d (supported: 128)", d->block_size);
  if (d->top_k != 16) return fail(MSA_ERR_UNSUPPORTED, "top_k=%d (supported: 16)", d->top_k);
  if (!pow2_upto32(d->num_kv_heads))
    return fail(MSA_ERR_UNSUPPORTED, "Hkv=%d (supported: powers of two up to 32)", d->num_kv_heads);
  if (d->num_q_heads / d->num_kv_heads > 16)
    return fail(MSA_ERR_UNSUPPORTED, "group size Hq/Hkv=%d (supported: <= 16)", d->num_q_heads / d->num_kv_heads);
  if (isnan(d->softmax_scale) || isinf(d->softmax_scale))
    return fail(MSA_ERR_BAD_SHAPE, "softmax_scale is not finite");
  return MSA_OK;
}

// Batch consistency from the host mirrors; `cache` may be NULL (no capacity check).
msa_status check_batch(const msa_dims* d, const msa_batch* b, const msa_cache* cache) {
  if (!b) return fail(MSA_ERR_NULL_POINTER, "batch is NULL");
  if (!b->seq_lens || !b->cu_q) return fail(MSA_ERR_NULL_POINTER, "batch device arrays are NULL");
  if (!b->seq_lens_host || !b->cu_q_host) return fail(MSA_ERR_NULL_POINTER, "batch host mirrors are NULL");
  if (b->num_seqs <= 0) return fail(MSA_ERR_BAD_SHAPE, "num_seqs=%d must be positive", b->num_seqs);
  if (b->total_q < 0) return fail(MSA_ERR_BAD_SHAPE, "total_q=%d is negative", b->total_q);
  if (b->cu_q_host[0] != 0) return fail(MSA_ERR_BAD_SHAPE, "cu_q[0]=%d must be 0", b->cu_q_host[0]);
  for (int s = 0; s < b->num_seqs; ++s) {
    const int nq = b->cu_q_host[s + 1] - b->cu_q_host[s];
    const int L = b->seq_lens_host[s];
    if (nq < 0) return fail(MSA_ERR_BAD_SHAPE, "cu_q decreases at sequence %d", s);
    if (L < 0 || nq > L) return fail(MSA_ERR_BAD_SHAPE, "sequence %d: %d queries but seq_len %d", s, nq, L);
    if (cache && (int64_t)L > (int64_t)cache->max_blocks_per_seq * 128)
      return fail(MSA_ERR_CAPACITY, "sequence %d: seq_len %d exceeds max_blocks_per_seq*128 = %lld", s, L,
                  (long long)cache->max_blocks_per_seq * 128);
  }
  if (b->cu_q_host[b->num_seqs] != b->total_q)
    return fail(MSA_ERR_BAD_SHAPE, "cu_q[num_seqs]=%d differs from total_q=%d", b->cu_q_host[b->num_seqs], b->total_q);
  // Selections are addressed as (row * Hkv + group) * 16 + slot in 32 bits.
  if ((int64_t)b->total_q * d->num_kv_heads * 16 >= (int64_t)1 << 31)
    return fail(MSA_ERR_CAPACITY, "total_q * Hkv * 16 overflows 32-bit indexing");
  return MSA_OK;
}

msa_status check_cache(const msa_cache* c) {
  if (!c) return fail(MSA_ERR_NULL_POINTER, "cache is NULL");
  if (!c->k || !c->v || !c->k_idx || !c->block_table) return fail(MSA_ERR_NULL_POINTER, "cache arrays are NULL");
  if (!aligned16(c->k) || !aligned16(c->v) || !aligned16(c->k_idx) || !aligned16(c->block_table))
    return fail(MSA_ERR_MISALIGNED, "cache arrays must be 16-byte aligned");
  if (c->num_blocks <= 0 || c->max_blocks_per_seq <= 0)
    return fail(MSA_ERR_BAD_SHAPE, "num_blocks=%d and max_blocks_per_seq=%d must be positive", c->num_blocks,
                c->max_blocks_per_seq);
  return MSA_OK;
}

msa_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(MSA_ERR_NULL_POINTER, "%s is NULL", name);
  if (!aligned16(p)) return fail(MSA_ERR_MISALIGNED, "%s is not 16-byte aligned", name);
  return MSA_OK;
}

// Largest ceil(seq_len / 128) over sequences that have queries.
int64_t max_query_blocks(const msa_batch* b) {
  int64_t m = 0;
  for (int s = 0; s < b->num_seqs; ++s)
    if (b->cu_q_host[s + 1] > b->cu_q_host[s]) m = std::max<int64_t>(m, (b->seq_lens_host[s] + 127) / 128);
  return m;
}

int max_q_per_seq(const msa_batch* b) {
  int m = 0;
  for (int s = 0; s < b->num_seqs; ++s) m = std::max(m, b->cu_q_host[s + 1] - b->cu_q_host[s]);
  return m;
}

msa::Problem make_problem(const msa_dims* d, const msa_batch* b, const msa_cache* c) {
  msa::Problem p{};
  p.hq = d->num_q_heads;
  p.hkv = d->num_kv_heads;
  p.head_dim = d->head_dim;
  p.index_dim = d->index_dim;
  p.group = d->num_q_heads / d->num_kv_heads;
  const double scale = d->softmax_scale > 0.f ? (double)d->softmax_scale : 1.0 / sqrt((double)d->head_dim);
  p.scale_log2e = (float)(scale * 1.4426950408889634);
  p.num_seqs = b->num_seqs;
  p.total_q = b->total_q;
  p.max_q_per_seq = max_q_per_seq(b);
  p.seq_lens = b->seq_lens;
  p.cu_q = b->cu_q;
  if (c) {
    p.k = static_cast<const uint16_t*>(c->k);
    p.v = static_cast<const uint16_t*>(c->v);
    p.k_idx = static_cast<const uint16_t*>(c->k_idx);
    p.block_table = c->block_table;
    p.num_blocks = c->num_blocks;
    p.max_blocks_per_seq = c->max_blocks_per_seq;
  }
  return p;
}

msa_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

#define MSA_TRY(expr)               \
  do {                              \
    const msa_status st_ = (expr);  \
    if (st_ != MSA_OK) return st_;  \
  } while (0)

msa_status check_prefill_capacity(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch) {
  if (cache->max_blocks_per_seq > msa::kMaxPrefillBlocks)
    return fail(MSA_ERR_CAPACITY, "prefill supports max_blocks_per_seq <= %d (got %d)", msa::kMaxPrefillBlocks,
                cache->max_blocks_per_seq);
  if ((int64_t)batch->num_seqs * dims->num_kv_heads * cache->max_blocks_per_seq >= (int64_t)1 << 31)
    return fail(MSA_ERR_CAPACITY, "num_seqs * Hkv * max_blocks_per_seq overflows 32-bit list ids");
  return MSA_OK;
}

msa_status check_one_query_per_sequence(const msa_batch* batch) {
  for (int s = 0; s < batch->num_seqs; ++s)
    if (batch->cu_q_host[s + 1] - batch->cu_q_host[s] != 1)
      return fail(MSA_ERR_BAD_SHAPE, "decode needs exactly one query per sequence (sequence %d has %d)", s,
                  batch->cu_q_host[s + 1] - batch->cu_q_host[s]);
  return MSA_OK;
}

msa_status check_attn(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch, const void* q,
                      const int32_t* sel, void* out) {
  MSA_TRY(check_dims(dims));
  MSA_TRY(check_cache(cache));
  MSA_TRY(check_batch(dims, batch, cache));
  MSA_TRY(check_ptr(q, "q"));
  MSA_TRY(check_ptr(sel, "sel"));
  MSA_TRY(check_ptr(out, "out"));
  return MSA_OK;
}

}  // namespace

extern "C" {

int32_t msa_abi_version(void) { return MSA_ABI_VERSION; }

const char* msa_last_error(void) { return g_last_error.c_str(); }

const char* msa_status_string(msa_status status) {
  // A C caller may pass any int: read the argument's bits instead of using a
  // value of enum type outside its enumerators' range.
  static_assert(sizeof(msa_status) == sizeof(int32_t), "msa_status is a 32-bit integer");
  int32_t code;
  memcpy(&code, &status, sizeof code);
  switch (code) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_NULL_POINTER: return "MSA_ERR_NULL_POINTER";
    case MSA_ERR_BAD_SHAPE: return "MSA_ERR_BAD_SHAPE";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED";
    case MSA_ERR_MISALIGNED: return "MSA_ERR_MISALIGNED";
    case MSA_ERR_CAPACITY: return "MSA_ERR_CAPACITY";
    case MSA_ERR_WORKSPACE: return "MSA_ERR_WORKSPACE";
    case MSA_ERR_HIP: return "MSA_ERR_HIP";
  }
  return "MSA_ERR_UNKNOWN";
}

msa_status msa_kv_append(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch, const void* k_new,
                         const void* v_new, const void* k_idx_new, void* stream) {
  MSA_TRY(check_dims(dims));
  MSA_TRY(check_cache(cache));
  MSA_TRY(check_batch(dims, batch, cache));
  MSA_TRY(check_ptr(k_new, "k_new"));
  MSA_TRY(check_ptr(v_new, "v_new"));
  MSA_TRY(check_ptr(k_idx_new, "k_idx_new"));
  const msa::Problem p = make_problem(dims, batch, cache);
  return hip_status(msa::launch_kv_append(p, static_cast<uint16_t*>(cache->k), static_cast<uint16_t*>(cache->v),
                                          static_cast<uint16_t*>(cache->k_idx), static_cast<const uint16_t*>(k_new),
                                          static_cast<const uint16_t*>(v_new),
                                          static_cast<const uint16_t*>(k_idx_new), max_q_per_seq(batch),
                                          static_cast<hipStream_t>(stream)),
                    "msa_kv_append launch");
}

msa_status msa_index_score(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch, const void* q_idx,
                           float* block_scores, int64_t ld, void* stream) {
  MSA_TRY(check_dims(dims));
  MSA_TRY(check_cache(cache));
  MSA_TRY(check_batch(dims, batch, cache));
  MSA_TRY(check_ptr(q_idx, "q_idx"));
  MSA_TRY(check_ptr(block_scores, "block_scores"));
  const int64_t need = max_query_blocks(batch);
  if (ld < need) return fail(MSA_ERR_BAD_SHAPE, "ld=%lld is less than the %lld blocks of the longest sequence",
                             (long long)ld, (long long)need);
  const msa::Problem p = make_problem(dims, batch, cache);
  return hip_status(msa::launch_index_score(p, static_cast<const uint16_t*>(q_idx), block_scores, ld,
                                            batch->seq_lens_host, batch->cu_q_host, static_cast<hipStream_t>(stream)),
                    "msa_index_score launch");
}

msa_status msa_block_topk(const msa_dims* dims, const msa_batch* batch, const float* block_scores, int64_t ld,
                          int32_t* sel, void* stream) {
  MSA_TRY(check_dims(dims));
  MSA_TRY(check_batch(dims, batch, nullptr));
  MSA_TRY(check_ptr(block_scores, "block_scores"));
  MSA_TRY(check_ptr(sel, "sel"));
  const int64_t need = max_query_blocks(batch);
  if (ld < need) return fail(MSA_ERR_BAD_SHAPE, "ld=%lld is less than the %lld blocks of the longest sequence",
                             (long long)ld, (long long)need);
  const msa::Problem p = make_problem(dims, batch, nullptr);
  return hip_status(msa::launch_block_topk(p, block_scores, ld, sel, need, static_cast<hipStream_t>(stream)),
                    "msa_block_topk launch");
}

msa_status msa_index_select(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch, const void* q_idx,
                            int32_t* sel, void* workspace, size_t ws_bytes, void* stream) {
  MSA_TRY(check_dims(dims));
  MSA_TRY(check_cache(cache));
  MSA_TRY(check_batch(dims, batch, cache));
  MSA_TRY(check_ptr(q_idx, "q_idx"));
  MSA_TRY(check_ptr(sel, "sel"));
  const int64_t ld = std::max<int64_t>(1, max_query_blocks(batch));
  const int64_t row_bytes = (int64_t)dims->num_kv_heads * ld * (int64_t)sizeof(float);
  if (!workspace || ws_bytes < (size_t)(kSelectMetaBytes + row_bytes))
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes given, at least %lld needed (one query row)",
                workspace ? ws_bytes : 0, (long long)(kSelectMetaBytes + row_bytes));
  if (!aligned16(workspace)) return fail(MSA_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  const msa::Problem p = make_problem(dims, batch, cache);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const auto* qi = static_cast<const uint16_t*>(q_idx);
  int32_t* meta = static_cast<int32_t*>(workspace);
  float* scores = reinterpret_cast<float*>(static_cast<char*>(workspace) + kSelectMetaBytes);
  // Rows per chunk: as many as the workspace holds pooled scores for.
  const int64_t cap = std::max<int64_t>(1, (int64_t)(ws_bytes - kSelectMetaBytes) / row_bytes);
  const int32_t* L = batch->seq_lens_host;
  const int32_t* cu = batch->cu_q_host;
  const int mbps = cache->max_blocks_per_seq;
  // Score + select one chunk whose rows are [row_lo, row_lo + pc.total_q) of the batch.
  auto run = [&](msa::Problem pc, const int32_t* lens_host, const int32_t* cu_host, int64_t row_lo,
                 int64_t max_blocks) -> hipError_t {
    // The chunk's pooled scores sit at the start of the workspace, its first row (row_lo) first;
    // q_idx and sel are addressed by the batch's own row numbers.
    hipError_t e = msa::launch_index_score(pc, qi, scores, ld, lens_host, cu_host, st, row_lo);
    if (e != hipSuccess) return e;
    return msa::launch_block_topk(pc, scores, ld, sel, max_blocks, st, row_lo);
  };
  int s = 0;
  while (s < batch->num_seqs) {
    const int nq = cu[s + 1] - cu[s];
    if (nq == 0) { ++s; continue; }
    if (nq > cap) {
      // One long sequence: row ranges of it, each a one-sequence sub-batch (a prefill chunk).
      for (int r0 = cu[s]; r0 < cu[s + 1]; r0 += (int)cap) {
        const int r1 = (int)std::min<int64_t>(cu[s + 1], r0 + cap);
        const int32_t len = L[s] - (cu[s + 1] - r1);  // the cache length seen by the chunk's last row
        const int32_t lens_host[1] = {len};
        const int32_t cu_host[2] = {r0, r1};
        hipError_t e = msa::launch_write_subbatch(meta, len, r0, r1, st);
        if (e != hipSuccess) return hip_status(e, "msa_index_select launch");
        msa::Problem pc = p;
        pc.num_seqs = 1;
        pc.total_q = r1 - r0;
        pc.max_q_per_seq = r1 - r0;
        pc.seq_lens = meta;
        pc.cu_q = meta + 1;
        pc.block_table = p.block_table + (int64_t)s * mbps;
        e = run(pc, lens_host, cu_host, r0, (len + 127) / 128);
        if (e != hipSuccess) return hip_status(e, "msa_index_select launch");
      }
      ++s;
      continue;
    }
    // Whole sequences while they fit: a sub-batch that points into the batch's own arrays.
    int s1 = s;
    int64_t rows = 0, max_blocks = 0;
    int max_q = 0;
    while (s1 < batch->num_seqs && rows + (cu[s1 + 1] - cu[s1]) <= cap) {
      rows += cu[s1 + 1] - cu[s1];
      max_q = std::max(max_q, cu[s1 + 1] - cu[s1]);
      if (cu[s1 + 1] > cu[s1]) max_blocks = std::max<int64_t>(max_blocks, (L[s1] + 127) / 128);
      ++s1;
    }
    msa::Problem pc = p;
    pc.num_seqs = s1 - s;
    pc.total_q = (int)rows;
    pc.max_q_per_seq = max_q;
    pc.seq_lens = batch->seq_lens + s;
    pc.cu_q = batch->cu_q + s;
    pc.block_table = p.block_table + (int64_t)s * mbps;
    const hipError_t e = run(pc, L + s, cu + s, cu[s], max_blocks);
    if (e != hipSuccess) return hip_status(e, "msa_index_select launch");
    s = s1;
  }
  return ok();
}

msa_status msa_block_attn_mass(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch, const void* q,
                               const int32_t* sel, const int32_t* rows, int32_t n_rows, float* mass, int64_t ld,
                               void* stream) {
  MSA_TRY(check_dims(dims));
  MSA_TRY(check_cache(cache));
  MSA_TRY(check_batch(dims, batch, cache));
  MSA_TRY(check_ptr(q, "q"));
  if (sel) MSA_TRY(check_ptr(sel, "sel"));
  MSA_TRY(check_ptr(rows, "rows"));
  MSA_TRY(check_ptr(mass, "mass"));
  if (n_rows < 0) return fail(MSA_ERR_BAD_SHAPE, "n_rows=%d is negative", n_rows);
  if ((int64_t)n_rows * dims->num_kv_heads > INT32_MAX)
    return fail(MSA_ERR_BAD_SHAPE, "n_rows * num_kv_heads exceeds 2^31 - 1");
  const int64_t need = max_query_blocks(batch);
  if (ld < need) return fail(MSA_ERR_BAD_SHAPE, "ld=%lld is less than the %lld blocks of the longest sequence",
                             (long long)ld, (long long)need);
  const msa::Problem p = make_problem(dims, batch, cache);
  return hip_status(msa::launch_block_attn_mass(p, static_cast<const uint16_t*>(q), sel, rows, n_rows, mass, ld,
                                                static_cast<hipStream_t>(stream)),
                    "msa_block_attn_mass launch");
}

msa_status msa_selection_quality(const msa_dims* dims, const msa_batch* batch, const int32_t* rows, int32_t n_rows,
                                 const float* mass, const float* sel_mass, const float* block_scores,
                                 const int32_t* sel, int64_t ld, float* quality, void* stream) {
  MSA_TRY(check_dims(dims));
  MSA_TRY(check_batch(dims, batch, nullptr));
  MSA_TRY(check_ptr(rows, "rows"));
  MSA_TRY(check_ptr(mass, "mass"));
  MSA_TRY(check_ptr(sel_mass, "sel_mass"));
  MSA_TRY(check_ptr(block_scores, "block_scores"));
  MSA_TRY(check_ptr(sel, "sel"));
  MSA_TRY(check_ptr(quality, "quality"));
  if (n_rows < 0) return fail(MSA_ERR_BAD_SHAPE, "n_rows=%d is negative", n_rows);
  if ((int64_t)n_rows * dims->num_kv_heads > INT32_MAX)
    return fail(MSA_ERR_BAD_SHAPE, "n_rows * num_kv_heads exceeds 2^31 - 1");
  const int64_t need = max_query_blocks(batch);
  if (ld < need) return fail(MSA_ERR_BAD_SHAPE, "ld=%lld is less than the %lld blocks of the longest sequence",
                             (long long)ld, (long long)need);
  const msa::Problem p = make_problem(dims, batch, nullptr);
  return hip_status(msa::launch_selection_quality(p, rows, n_rows, mass, sel_mass, block_scores, sel, ld, quality,
                                                  static_cast<hipStream_t>(stream)),
                    "msa_selection_quality launch");
}

msa_status msa_dense_attn_prefill(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch,
                                  const void* q, void* out, void* stream) {
  MSA_TRY(check_dims(dims));
  MSA_TRY(check_cache(cache));
  MSA_TRY(check_batch(dims, batch, cache));
  MSA_TRY(check_ptr(q, "q"));
  MSA_TRY(check_ptr(out, "out"));
  const msa::Problem p = make_problem(dims, batch, cache);
  return hip_status(msa::launch_dense_prefill(p, static_cast<const uint16_t*>(q), static_cast<uint16_t*>(out),
                                              static_cast<hipStream_t>(stream)),
                    "msa_dense_attn_prefill launch");
}

msa_status msa_dense_attn_decode(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch,
                                 const void* q, void* out, void* workspace, size_t ws_bytes, void* stream) {
  MSA_TRY(check_dims(dims));
  MSA_TRY(check_cache(cache));
  MSA_TRY(check_batch(dims, batch, cache));
  MSA_TRY(check_ptr(q, "q"));
  MSA_TRY(check_ptr(out, "out"));
  MSA_TRY(check_one_query_per_sequence(batch));
  const msa::Problem p = make_problem(dims, batch, cache);
  const int max_blocks = (int)max_query_blocks(batch);
  const size_t need = msa::dense_decode_workspace_bytes(p, max_blocks);
  if (!workspace || ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? ws_bytes : 0, need);
  if (!aligned16(workspace)) return fail(MSA_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  return hip_status(msa::launch_dense_decode(p, static_cast<const uint16_t*>(q), static_cast<uint16_t*>(out),
                                             workspace, max_blocks, static_cast<hipStream_t>(stream)),
                    "msa_dense_attn_decode launch");
}

size_t msa_workspace_size(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch, int32_t call) {
  if (check_dims(dims) != MSA_OK || check_cache(cache) != MSA_OK || check_batch(dims, batch, cache) != MSA_OK)
    return 0;
  const msa::Problem p = make_problem(dims, batch, cache);
  switch (call) {
    case MSA_CALL_SPARSE_ATTN_PREFILL:
      if (check_prefill_capacity(dims, cache, batch) != MSA_OK) return 0;
      ok();
      return msa::prefill_workspace_bytes(p);
    case MSA_CALL_SPARSE_ATTN_PREFILL_PLAN:
      if (check_prefill_capacity(dims, cache, batch) != MSA_OK) return 0;
      ok();
      return msa::prefill_plan_bytes(p);
    case MSA_CALL_SPARSE_ATTN_PREFILL_RUN:
      if (check_prefill_capacity(dims, cache, batch) != MSA_OK) return 0;
      ok();
      return msa::prefill_run_bytes(p);
    case MSA_CALL_SPARSE_ATTN_DECODE: ok(); return msa::decode_workspace_bytes(p);
    case MSA_CALL_DENSE_ATTN_DECODE: ok(); return msa::dense_decode_workspace_bytes(p, (int)max_query_blocks(batch));
    case MSA_CALL_DECODE_STEP: ok(); return msa::decode_step_workspace_bytes(p);
    case MSA_CALL_INDEX_SELECT: {
      ok();
      const int64_t ld = std::max<int64_t>(1, max_query_blocks(batch));
      const int64_t row_bytes = (int64_t)dims->num_kv_heads * ld * (int64_t)sizeof(float);
      const int64_t rows = std::max<int64_t>(1, std::min<int64_t>(batch->total_q, kSelectScoresBudget / row_bytes));
      return (size_t)(kSelectMetaBytes + rows * row_bytes);
    }
  }
  fail(MSA_ERR_BAD_SHAPE, "unknown call id %d", call);
  return 0;
}

msa_status msa_sparse_attn_prefill(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch, const void* q,
                                   const int32_t* sel, void* out, void* workspace, size_t ws_bytes, void* stream) {
  MSA_TRY(check_attn(dims, cache, batch, q, sel, out));
  MSA_TRY(check_prefill_capacity(dims, cache, batch));
  const msa::Problem p = make_problem(dims, batch, cache);
  const size_t need = msa::prefill_workspace_bytes(p);
  if (!workspace || ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? ws_bytes : 0, need);
  if (!aligned16(workspace)) return fail(MSA_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  return hip_status(msa::launch_attn_prefill(p, static_cast<const uint16_t*>(q), sel, static_cast<uint16_t*>(out),
                                             workspace, static_cast<hipStream_t>(stream)),
                    "msa_sparse_attn_prefill launch");
}

msa_status msa_sparse_attn_prefill_plan(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch,
                                        const int32_t* sel, void* plan, size_t plan_bytes, void* stream) {
  MSA_TRY(check_dims(dims));
  MSA_TRY(check_cache(cache));
  MSA_TRY(check_batch(dims, batch, cache));
  MSA_TRY(check_ptr(sel, "sel"));
  MSA_TRY(check_prefill_capacity(dims, cache, batch));
  const msa::Problem p = make_problem(dims, batch, cache);
  const size_t need = msa::prefill_plan_bytes(p);
  if (!plan || plan_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "plan buffer of %zu bytes given, %zu needed", plan ? plan_bytes : 0, need);
  if (!aligned16(plan)) return fail(MSA_ERR_MISALIGNED, "plan is not 16-byte aligned");
  return hip_status(msa::launch_attn_prefill_plan(p, sel, plan, static_cast<hipStream_t>(stream)),
                    "msa_sparse_attn_prefill_plan launch");
}

msa_status msa_sparse_attn_prefill_run(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch,
                                       const void* q, const int32_t* sel, const void* plan, void* out,
                                       void* workspace, size_t ws_bytes, void* stream) {
  MSA_TRY(check_attn(dims, cache, batch, q, sel, out));
  MSA_TRY(check_ptr(plan, "plan"));
  MSA_TRY(check_prefill_capacity(dims, cache, batch));
  const msa::Problem p = make_problem(dims, batch, cache);
  const size_t need = msa::prefill_run_bytes(p);
  if (!workspace || ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? ws_bytes : 0, need);
  if (!aligned16(workspace)) return fail(MSA_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  return hip_status(msa::launch_attn_prefill_run(p, static_cast<const uint16_t*>(q), sel, plan,
                                                 static_cast<uint16_t*>(out), workspace,
                                                 static_cast<hipStream_t>(stream)),
                    "msa_sparse_attn_prefill_run launch");
}

msa_status msa_sparse_attn_decode(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch, const void* q,
                                  const int32_t* sel, void* out, void* workspace, size_t ws_bytes, void* stream) {
  MSA_TRY(check_attn(dims, cache, batch, q, sel, out));
  MSA_TRY(check_one_query_per_sequence(batch));
  const msa::Problem p = make_problem(dims, batch, cache);
  const size_t need = msa::decode_workspace_bytes(p);
  if (!workspace || ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? ws_bytes : 0, need);
  if (!aligned16(workspace)) return fail(MSA_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  return hip_status(msa::launch_attn_decode(p, static_cast<const uint16_t*>(q), sel, static_cast<uint16_t*>(out),
                                            workspace, static_cast<hipStream_t>(stream)),
                    "msa_sparse_attn_decode launch");
}

msa_status msa_decode_step(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch, const void* k_new,
                           const void* v_new, const void* k_idx_new, const void* q_idx, const void* q,
                           float* block_scores, int64_t ld, int32_t* sel, void* out, void* workspace,
                           size_t ws_bytes, void* stream) {
  MSA_TRY(check_dims(dims));
  MSA_TRY(check_cache(cache));
  MSA_TRY(check_batch(dims, batch, cache));
  MSA_TRY(check_one_query_per_sequence(batch));
  MSA_TRY(check_ptr(k_new, "k_new"));
  MSA_TRY(check_ptr(v_new, "v_new"));
  MSA_TRY(check_ptr(k_idx_new, "k_idx_new"));
  MSA_TRY(check_ptr(q_idx, "q_idx"));
  MSA_TRY(check_ptr(q, "q"));
  MSA_TRY(check_ptr(block_scores, "block_scores"));
  MSA_TRY(check_ptr(sel, "sel"));
  MSA_TRY(check_ptr(out, "out"));
  const int64_t need_ld = max_query_blocks(batch);
  if (ld < need_ld) return fail(MSA_ERR_BAD_SHAPE, "ld=%lld is less than the %lld blocks of the longest sequence",
                                (long long)ld, (long long)need_ld);
  const msa::Problem p = make_problem(dims, batch, cache);
  const size_t need = msa::decode_step_workspace_bytes(p);
  if (!workspace || ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? ws_bytes : 0, need);
  if (!aligned16(workspace)) return fail(MSA_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = msa::launch_decode_append_score(
      p, static_cast<uint16_t*>(cache->k), static_cast<uint16_t*>(cache->v), static_cast<uint16_t*>(cache->k_idx),
      static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
      static_cast<const uint16_t*>(k_idx_new), static_cast<const uint16_t*>(q_idx), block_scores, ld,
      msa::decode_step_counters(p, workspace), batch->seq_lens_host, batch->cu_q_host, st);
  if (e != hipSuccess) return hip_status(e, "msa_decode_step launch (append and scoring)");
  return hip_status(msa::launch_decode_step_attn(p, static_cast<const uint16_t*>(q), block_scores, ld, sel,
                                                 static_cast<uint16_t*>(out), workspace, need_ld, st),
                    "msa_decode_step launch (selection and attention)");
}

msa_status msa_sparse_attn_decode_noalloc(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch,
                                          const void* q, const int32_t* sel, void* out, void* stream) {
  MSA_TRY(check_attn(dims, cache, batch, q, sel, out));
  MSA_TRY(check_one_query_per_sequence(batch));
  const msa::Problem p = make_problem(dims, batch, cache);
  const size_t need = msa::decode_scratch_need(p);
  if (need > msa::decode_scratch_capacity())
    return fail(MSA_ERR_WORKSPACE, "this decode needs %zu bytes of scratch; the library's static scratch holds %zu",
                need, msa::decode_scratch_capacity());
  const hipStream_t st = static_cast<hipStream_t>(stream);
  int device = 0;
  hipError_t e = st ? hipStreamGetDevice(st, &device) : hipGetDevice(&device);
  if (e != hipSuccess) return hip_status(e, "msa_sparse_attn_decode_noalloc: device of the stream");
  void* ws = nullptr;
  if ((e = msa::decode_scratch(device, &ws)) != hipSuccess)
    return hip_status(e, "msa_sparse_attn_decode_noalloc: scratch address");
  return hip_status(msa::launch_attn_decode(p, static_cast<const uint16_t*>(q), sel, static_cast<uint16_t*>(out), ws,
                                            st),
                    "msa_sparse_attn_decode_noalloc launch");
}

}  // extern "C"
