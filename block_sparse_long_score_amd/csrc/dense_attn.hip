// dense_attn.hip — dense causal GQA softmax attention over the block-major
// KV cache: every query row attends to all keys at or before its position.
//
// Source: "MiniMax 模型迭代与竞品分析：从 Text-01、M1、M2 到 M3", §2: the
// softmax-attention equation (scores q.k/sqrt(d_k), causal, softmax over the
// attended keys, probability-weighted sum of values) and, in §2-§3, the
// layers and the training warmup that run full attention beside the sparse
// ones.  It is MSA with every causal block selected, on the cache MSA uses.
//
// Schedule (queries outer).  One workgroup of 4 waves per (sequence, tile of
// 128 query rows, query head); wave w owns 32 consecutive rows.  The
// workgroup walks the causal blocks in order, stages each block's K and V^T
// in LDS (shared by the 4 waves) and every wave runs its rows against it on
// the 32x32x16 bf16 MFMA (the tile pieces of attn_tiles.h), with an online
// softmax in base 2.  Only the one or two blocks that hold the tile's own
// positions are masked.  The running maximum is raised only when a block's
// maximum exceeds it by more than 2^8, so the accumulators are rescaled
// rarely; numerator and denominator share the reference value, so the
// result is unchanged.
//
// Work order.  Workgroups are dispatched round-robin over the 8 XCDs
// (workgroup i runs on XCD i % 8), each with its own L2.  The mapping from
// workgroup id to (tile, sequence, head) puts all heads of one KV group, for
// the same tiles, on the same XCD, so they read the group's K/V blocks from
// that XCD's L2 at about the same time; tiles run latest positions first
// (the longest rows first) for load balance.
#include "attn_tiles.h"
#include "msa_kernels.h"

namespace msa {

constexpr int kDenseRows = 128;  // query rows of one head per workgroup

struct DenseArgs {
  Problem p;
  const uint16_t* q;
  uint16_t* out;
  int n_tf;  // row tiles of the longest query range
};

// Workgroup id -> (tile counted from the end of the sequence's query rows,
// sequence, query head).  False if the id names no work.
__device__ __forceinline__ bool dense_item(const DenseArgs& a, int& tf, int& s, int& h) {
  const Problem& p = a.p;
  const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
  const int S = p.num_seqs, G = p.group;
  int g, j;
  if (p.hkv >= 8) {  // hkv/8 groups per XCD
    const int gx = p.hkv >> 3;
    const int per = S * gx * G;
    tf = k / per;
    int rem = k - tf * per;
    s = rem / (gx * G);
    rem -= s * gx * G;
    const int m = rem / G;
    j = rem - m * G;
    g = x + 8 * m;
  } else {  // 8/hkv XCDs per group, tiles dealt round-robin between them
    const int R = 8 / p.hkv;
    g = x & (p.hkv - 1);
    const int sub = x / p.hkv;
    const int tq = k / (S * G);
    const int rem = k - tq * S * G;
    s = rem / G;
    j = rem - s * G;
    tf = tq * R + sub;
  }
  h = g * G + j;
  return tf < a.n_tf;
}

template <int D>
__global__ __launch_bounds__(256, 2) void dense_prefill_kernel(DenseArgs a) {
  __shared__ Lds<D> sm;
  const Problem& p = a.p;
  int tf, s, h;
  if (!dense_item(a, tf, s, h)) return;
  const int q_beg = p.cu_q[s], q_end = p.cu_q[s + 1];
  const int r_hi = q_end - kDenseRows * tf;  // rows [r_hi - 128, r_hi) of which those >= q_beg exist
  if (r_hi <= q_beg) return;
  const int g = h / p.group;
  const int seq_len = p.seq_lens[s];
  const int nb = ((seq_len - 1 - kDenseRows * tf) >> 7) + 1;  // blocks up to the tile's last position
  const int32_t* bt = p.block_table + (int64_t)s * p.max_blocks_per_seq;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int row0 = r_hi - kDenseRows + 32 * wave;  // this wave's first (possibly absent) row
  const int my_row = max(row0 + l32, q_beg);       // rows before the sequence's queries stand in for its first
  const int t = seq_len - (q_end - my_row);        // this lane's query position
  const int t_first = seq_len - (q_end - max(row0, q_beg));
  const int t_last = seq_len - (q_end - (row0 + 31));
  const bool active = row0 + 31 >= q_beg;          // wave has rows of its own
  const int last_b = active ? t_last >> 7 : -1;
  const int first_masked = t_first >> 7;

  bf16x8 bq[D / 16];
  {
    QRaw<D> raw;
    load_q_raw<D>(a.q + ((int64_t)my_row * p.hq + h) * D, raw);
    q_operand<D>(raw, bq);
  }
  const float c = p.scale_log2e;
  float m = -1e30f, l = 0.f;  // finite start: exp2(-inf - m) = 0 for masked keys
  f32x16 oacc[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n)
    oacc[n] = f32x16{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

  for (int b = 0; b < nb; ++b) {
    const int phys = bt[b];
    if (phys < 0 || phys >= p.num_blocks) continue;  // absent blocks hold no keys (same for the whole workgroup)
    __syncthreads();  // previous block no longer read
    const int64_t base = ((int64_t)phys * kBlock * p.hkv + g) * D;
    stage_block<D>(sm, p.k + base, p.v + base, (int64_t)p.hkv * D, min(kBlock, seq_len - b * kBlock));
    __syncthreads();
    if (b > last_b) continue;

    f32x16 sacc[4];
    block_scores<D>(sm, bq, sacc);
    if (b >= first_masked) {  // keys after some row's position
      const int lim = t - b * kBlock;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = t4 * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          sacc[t4][i] = key <= lim ? sacc[t4][i] : -__builtin_inff();
        }
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[t4][i]);
    mx = fmaxf(mx, swap_halves(mx)) * c;
    const bool grow = mx > m + 8.f;
    if (__ballot(grow) != 0) {
      const float mn = grow ? mx : m;
      const float alpha = fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int n = 0; n < D / 32; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[n][i] *= alpha;
      m = mn;
    }
    float sum = 0.f;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(fmaf(sacc[t4][i], c, -m));
        sacc[t4][i] = e;
        sum += e;
      }
    l += sum + swap_halves(sum);
    block_pv<D, true>(sm, sacc, oacc);
  }
  if (!active) return;

  // Output rows in natural dim order, 64-byte row segments (the partial-row
  // store of the Main Branch): lane (row rho, half hf) holds dims
  // 32n + 8*(i/4) + 4hf + (i%4); a swap across the wave halves and one with
  // the lane 16 away give four lanes 32 consecutive dims of one row.
  const float inv_l = 1.0f / l;
  const int a16 = l32 >> 4, b16 = l32 & 15;
  const bool okA = row0 + b16 >= q_beg, okB = row0 + 16 + b16 >= q_beg;
  uint16_t* dstA = a.out + ((int64_t)(row0 + b16) * p.hq + h) * D + 8 * half + 16 * a16;
  uint16_t* dstB = a.out + ((int64_t)(row0 + 16 + b16) * p.hq + h) * D + 8 * half + 16 * (1 - a16);
#pragma unroll
  for (int n = 0; n < D / 32; ++n) {
    const f32x16& o = oacc[n];
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = pack_bf16x2(o[2 * i] * inv_l, o[2 * i + 1] * inv_l);
    const auto s0 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
    const auto s2 = __builtin_amdgcn_permlane32_swap(w[4], w[6], false, false);
    const auto s3 = __builtin_amdgcn_permlane32_swap(w[5], w[7], false, false);
    const u32x4 c1{s0[0], s1[0], s0[1], s1[1]};
    u32x4 c2{s2[0], s3[0], s2[1], s3[1]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto sw = __builtin_amdgcn_permlane16_swap(c2[i], c2[i], false, false);
      c2[i] = a16 ? sw[0] : sw[1];
    }
    if (okA) store16(dstA + 32 * n, a16 ? c2 : c1);
    if (okB) store16(dstB + 32 * n, a16 ? c1 : c2);
  }
}

int64_t dense_prefill_grid(const Problem& p) {
  const int64_t n_tf = (p.max_q_per_seq + kDenseRows - 1) / kDenseRows;
  if (p.hkv >= 8) return n_tf * p.num_seqs * p.hq;
  const int64_t R = 8 / p.hkv;
  return 8 * ((n_tf + R - 1) / R) * p.num_seqs * p.group;
}

hipError_t launch_dense_prefill(const Problem& p, const uint16_t* q, uint16_t* out, hipStream_t stream) {
  if (p.total_q == 0) return hipSuccess;
  const DenseArgs a{p, q, out, (p.max_q_per_seq + kDenseRows - 1) / kDenseRows};
  const dim3 grid((unsigned)dense_prefill_grid(p));
  if (p.head_dim == 128)
    hipLaunchKernelGGL(dense_prefill_kernel<128>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(dense_prefill_kernel<64>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace msa
