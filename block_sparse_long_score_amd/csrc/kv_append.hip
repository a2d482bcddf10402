// kv_append.hip — write this step's new tokens into the block-major cache.
//
// Source: "前沿架构解码手记（三）：MiniMax M2.7 → M3", §2.1 (KV-Block-Major):
// the cache nests block -> token -> head -> dim, so one token's K (all heads)
// is one contiguous run of Hkv*D values inside its block, and a block is one
// contiguous run of 128 such tokens.  Keys/values of past tokens are cached;
// queries are not ("MiniMax 模型迭代与竞品分析" §2, Q/K/V paragraph).
//
// Pure copy: every thread moves 16-byte vectors; one grid row per sequence.
#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {

struct AppendArgs {
  Problem p;
  uint16_t* k_cache;
  uint16_t* v_cache;
  uint16_t* k_idx_cache;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const uint16_t* k_idx_new;
};

__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  const Problem& p = a.p;
  const int s = blockIdx.y;
  const int row0 = p.cu_q[s];
  const int nq = p.cu_q[s + 1] - row0;
  const int first_pos = p.seq_lens[s] - nq;
  const int kv_vec = (p.hkv * p.head_dim) >> 3;  // 16-byte vectors per token of K (and of V)
  const int ki_vec = p.index_dim >> 3;           // 16-byte vectors per token of K_idx
  const int per_tok = 2 * kv_vec + ki_vec;
  const int64_t total = (int64_t)nq * per_tok;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int i = (int)(idx / per_tok);
    int vec = (int)(idx - (int64_t)i * per_tok);
    const int pos = first_pos + i;
    const int phys = p.block_table[(int64_t)s * p.max_blocks_per_seq + (pos >> 7)];
    if (phys < 0 || phys >= p.num_blocks) continue;
    const int64_t slot = (int64_t)phys * kBlock + (pos & 127);
    const int64_t row = row0 + i;
    if (vec < kv_vec) {
      store16(a.k_cache + (slot * kv_vec + vec) * 8, load16(a.k_new + (row * kv_vec + vec) * 8));
    } else if ((vec -= kv_vec) < kv_vec) {
      store16(a.v_cache + (slot * kv_vec + vec) * 8, load16(a.v_new + (row * kv_vec + vec) * 8));
    } else {
      vec -= kv_vec;
      store16(a.k_idx_cache + (slot * ki_vec + vec) * 8, load16(a.k_idx_new + (row * ki_vec + vec) * 8));
    }
  }
}

hipError_t launch_kv_append(const Problem& p, uint16_t* k_cache, uint16_t* v_cache, uint16_t* k_idx_cache,
                            const uint16_t* k_new, const uint16_t* v_new, const uint16_t* k_idx_new,
                            int max_q_per_seq, hipStream_t stream) {
  if (max_q_per_seq <= 0 || p.num_seqs <= 0) return hipSuccess;
  const int64_t per_tok = 2 * ((p.hkv * p.head_dim) >> 3) + (p.index_dim >> 3);
  const int64_t work = (int64_t)max_q_per_seq * per_tok;
  int64_t blocks = (work + 255) / 256;
  int64_t cap = 32768 / p.num_seqs;  // bound the grid; the kernel strides over the rest
  if (cap < 1) cap = 1;
  if (blocks > cap) blocks = cap;
  AppendArgs a{p, k_cache, v_cache, k_idx_cache, k_new, v_new, k_idx_new};
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks, (unsigned)p.num_seqs), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace msa
