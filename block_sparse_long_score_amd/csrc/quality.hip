// quality.hip — selection quality of MSA against dense attention.
//
// Source: "MiniMax 模型迭代与竞品分析：从 Text-01、M1、M2 到 M3", §2.  The
// indexer is trained by aligning its block distribution Q with the Main
// Branch's group-averaged importance P over the candidate blocks with
// D_KL(P || Q), and MSA is to be judged not only by speed but by selection
// recall and by how much of the attention score the chosen blocks cover.
//
// block_mass_kernel: per-block attention mass for sampled query rows, over
// one of two token sets: every causal token (the dense mass, for coverage
// and recall), or the tokens of the row's selected blocks (the Main Branch's
// own softmax: P of the KL, over the candidate blocks).  One workgroup per
// (sampled row, group); its waves (4, or 16 for small samples) take the
// blocks round-robin.  Scores of the group's heads use the 16x16x32 bf16 MFMA
// with 16 keys on M (K rows read straight from the block-major cache) and the
// heads on N (padded to 16), so lane (head l%16, quarter l/16) holds 4 keys
// of one head per key tile.  Pass 1 forms each head's softmax max and sum
// over the token set (online, in base 2); pass 2 recomputes the scores and
// sums exp2(z - max) / sum over each block's tokens and over the group's
// heads.
//
// selection_quality_kernel: one wave per (sampled row, group): coverage of
// the selected blocks and recall of the top blocks by dense mass (exact K-th
// largest mass found bit by bit with wave ballots, equal masses to the lower
// index), and D_KL(P || Q) over the selected blocks, Q the softmax of their
// pooled index scores.
#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {

struct MassArgs {
  Problem p;
  const uint16_t* q;
  const int32_t* sel;  // NULL: every causal token; else the tokens of the row's selected blocks
  const int32_t* rows;
  int32_t n_rows;
  float* mass;
  int64_t ld;
  int hkv_shift;
};

__device__ __forceinline__ float sum_quarters(float v) {  // lanes l, l^16, l^32, l^48
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

__device__ __forceinline__ float max_quarters(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}

template <int D, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void block_mass_kernel(MassArgs a) {
  constexpr int KS = D / 32;
  __shared__ float st_s[WAVES][16][2];
  const Problem& p = a.p;
  const int G = p.group;
  const int k = blockIdx.x >> a.hkv_shift;
  const int g = blockIdx.x & ((1 << a.hkv_shift) - 1);
  const int r = a.rows[k];
  if (r < 0 || r >= p.total_q) return;
  const int s = seq_of_row(p.cu_q, p.num_seqs, r);
  const int t = p.seq_lens[s] - (p.cu_q[s + 1] - r);
  const int c = t >> 7;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, q4 = lane >> 4;
  const float cl = p.scale_log2e;

  // Q operand: head l16 of the group (zeros beyond G), dims 32*ks + 8*q4 .. +7.
  const bool head_ok = l16 < G;
  const uint16_t* qh = a.q + ((int64_t)r * p.hq + g * G + (head_ok ? l16 : 0)) * D + q4 * 8;
  bf16x8 bq[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const u32x4 x = load16(qh + ks * 32);
    bq[ks] = as_bf16x8(head_ok ? x : u32x4{0u, 0u, 0u, 0u});
  }
  const int64_t key_stride = (int64_t)p.hkv * D;
  const int32_t* table = p.block_table + (int64_t)s * p.max_blocks_per_seq;
  float* out = a.mass + ((int64_t)k * p.hkv + g) * a.ld;
  // The blocks of the token set: causal blocks 0..c, or the row's selected
  // slots (ids outside 0..c and unmapped blocks hold no keys).  Work item i of
  // n_items is block i, or the block of slot i.
  const int32_t* sel_row = a.sel ? a.sel + (((int64_t)r << a.hkv_shift) + g) * kTopK : nullptr;
  const int n_items = a.sel ? kTopK : c + 1;
  auto block_of = [&](int i) -> int { return sel_row ? sel_row[i] : i; };
  if (sel_row) {  // blocks that are not selected carry no mass
    for (int b = threadIdx.x; b <= c; b += blockDim.x) out[b] = 0.f;
    __syncthreads();
  }

  // Base-2 scaled scores of key tile kt of a block with nvalid causal keys:
  // lane (head l16, q4) gets keys 16*kt + 4*q4 + i; keys past nvalid are -inf.
  auto tile_scores = [&](const uint16_t* kb, int kt, int nvalid) -> f32x4 {
    const int key = kt * 16 + l16;
    const uint16_t* krow = kb + (int64_t)min(key, nvalid - 1) * key_stride + q4 * 8;
    bf16x8 ak[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ak[ks] = as_bf16x8(load16(krow + ks * 32));
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[ks], bq[ks], sc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = kt * 16 + 4 * q4 + i < nvalid ? sc[i] * cl : -__builtin_inff();
    return sc;
  };

  // Pass 1: per head, max and sum of 2^z over every token of the set.
  float m = -__builtin_inff(), l = 0.f;
  for (int i = wave; i < n_items; i += WAVES) {
    const int b = block_of(i);
    if (b < 0 || b > c) continue;
    const int phys = table[b];
    if (phys < 0 || phys >= p.num_blocks) continue;
    const uint16_t* kb = p.k + ((int64_t)phys * kBlock * p.hkv + g) * D;
    const int nvalid = b < c ? kBlock : t - b * kBlock + 1;
    for (int kt = 0; kt * 16 < nvalid; ++kt) {
      const f32x4 sc = tile_scores(kb, kt, nvalid);
      const float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      if (mx > -__builtin_inff()) {
        const float mn = fmaxf(m, mx);
        l = l * fast_exp2(m - mn) + fast_exp2(sc[0] - mn) + fast_exp2(sc[1] - mn) + fast_exp2(sc[2] - mn) +
            fast_exp2(sc[3] - mn);
        m = mn;
      }
    }
  }
  {
    const float mw = max_quarters(m);
    const float lw = sum_quarters(m > -__builtin_inff() ? l * fast_exp2(m - mw) : 0.f);
    if (q4 == 0) {
      st_s[wave][l16][0] = mw;
      st_s[wave][l16][1] = lw;
    }
  }
  __syncthreads();
  float M = -__builtin_inff();
#pragma unroll
  for (int w = 0; w < WAVES; ++w) M = fmaxf(M, st_s[w][l16][0]);
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    const float mw = st_s[w][l16][0];
    L += mw > -__builtin_inff() ? st_s[w][l16][1] * fast_exp2(mw - M) : 0.f;
  }
  const float inv_l = 1.0f / L;

  // Pass 2: mass of each block, summed over the group's heads.
  for (int i = wave; i < n_items; i += WAVES) {
    const int b = block_of(i);
    if (b < 0 || b > c) continue;
    const int phys = table[b];
    if (phys < 0 || phys >= p.num_blocks) continue;
    const uint16_t* kb = p.k + ((int64_t)phys * kBlock * p.hkv + g) * D;
    const int nvalid = b < c ? kBlock : t - b * kBlock + 1;
    float acc = 0.f;
    for (int kt = 0; kt * 16 < nvalid; ++kt) {
      const f32x4 sc = tile_scores(kb, kt, nvalid);
      acc += fast_exp2(sc[0] - M) + fast_exp2(sc[1] - M) + fast_exp2(sc[2] - M) + fast_exp2(sc[3] - M);
    }
    const float per_head = sum_quarters(acc) * inv_l;  // every lane takes part in the shuffles
    float v = head_ok ? per_head : 0.f;
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    if (lane == 0) out[b] = v / (float)G;
  }
}

struct QualityArgs {
  Problem p;
  const int32_t* rows;
  int32_t n_rows;
  const float* mass;      // dense mass per block (coverage, recall)
  const float* sel_mass;  // the Main Branch's mass over the selected blocks (P of the KL)
  const float* scores;
  const int32_t* sel;
  int64_t ld;
  float* quality;
  int hkv_shift;
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__global__ __launch_bounds__(256) void selection_quality_kernel(QualityArgs a) {
  const Problem& p = a.p;
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // sampled row k, group g
  if (w >= ((int64_t)a.n_rows << a.hkv_shift)) return;
  const int k = (int)(w >> a.hkv_shift);
  const int g = (int)(w & ((1 << a.hkv_shift) - 1));
  const int r = a.rows[k];
  if (r < 0 || r >= p.total_q) return;
  const int s = seq_of_row(p.cu_q, p.num_seqs, r);
  const int t = p.seq_lens[s] - (p.cu_q[s + 1] - r);
  const int n = (t >> 7) + 1;  // causal blocks 0..c
  const int64_t row = ((int64_t)r << a.hkv_shift) + g;
  const float* P = a.mass + w * a.ld;
  const float* S = a.scores + row * a.ld;

  // Coverage: mass on the selected blocks.
  const int bj = lane < kTopK ? a.sel[row * kTopK + lane] : -1;
  const bool sel_ok = bj >= 0 && bj < n;
  const float coverage = wave_sum(sel_ok ? P[bj] : 0.f);

  // Recall: T = the K-th largest mass key among the n blocks (key 0 marks
  // lanes past the end; every real mass is >= 0 and has a larger key).
  const int K = min(kTopK, n);
  auto key_at = [&](int b) -> uint32_t { return b < n ? order_key(P[b]) : 0u; };
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int cnt = 0;
    for (int j0 = 0; j0 < n; j0 += 64) cnt += __popcll(__ballot(key_at(j0 + lane) >= cand));
    if (cnt >= K) T = cand;
  }
  int gt = 0, eq_below = 0;
  for (int j0 = 0; j0 < n; j0 += 64) {
    const uint32_t key = key_at(j0 + lane);
    gt += __popcll(__ballot(key > T));
    const uint64_t eq = __ballot(key == T);
    if (sel_ok) {
      if (bj >= j0 + 64)
        eq_below += __popcll(eq);
      else if (bj >= j0)
        eq_below += __popcll(eq & ((1ull << (bj - j0)) - 1ull));
    }
  }
  const int need = K - gt;  // blocks equal to T that belong to the top K (the lowest indices)
  const uint32_t kb = sel_ok ? order_key(P[bj]) : 0u;
  const bool member = sel_ok && (kb > T || (kb == T && eq_below < need));
  const float recall = (float)__popcll(__ballot(member)) / (float)K;

  // D_KL(P || Q) over the selected blocks (lane j < 16 holds slot j): P the
  // Main Branch's mass, Q the softmax of the pooled scores over the same
  // blocks.  KL = sum P ln P - sum P S + lse(S) * sum P, over blocks with
  // P > 0 (an unmapped block has P = 0 and score -inf: Q = 0, no term).
  const float pb = sel_ok ? a.sel_mass[w * a.ld + bj] : 0.f;
  const float sb = sel_ok ? S[bj] : -__builtin_inff();
  const float smax = wave_max(sb);
  const float se = wave_sum(sel_ok && sb > -__builtin_inff() ? expf(sb - smax) : 0.f);
  const float spl = wave_sum(pb > 0.f ? pb * logf(pb) : 0.f);
  const float sps = wave_sum(pb > 0.f ? pb * sb : 0.f);
  const float sp = wave_sum(pb > 0.f ? pb : 0.f);
  const float kl = sp > 0.f ? spl - sps + (smax + logf(se)) * sp : 0.f;
  if (lane == 0) {
    float* q = a.quality + w * 3;
    q[0] = coverage;
    q[1] = recall;
    q[2] = kl;
  }
}

hipError_t launch_block_attn_mass(const Problem& p, const uint16_t* q, const int32_t* sel, const int32_t* rows,
                                  int32_t n_rows, float* mass, int64_t ld, hipStream_t stream) {
  int hkv_shift = 0;
  while ((1 << hkv_shift) < p.hkv) ++hkv_shift;
  if (n_rows == 0) return hipSuccess;
  MassArgs a{p, q, sel, rows, n_rows, mass, ld, hkv_shift};
  const int64_t pairs = (int64_t)n_rows << hkv_shift;
  const dim3 grid((unsigned)pairs);
  // Few (row, group) pairs (decode-sized samples): 16 waves each to keep enough loads in flight.
  if (pairs < 512) {
    if (p.head_dim == 128)
      hipLaunchKernelGGL((block_mass_kernel<128, 16>), grid, dim3(1024), 0, stream, a);
    else
      hipLaunchKernelGGL((block_mass_kernel<64, 16>), grid, dim3(1024), 0, stream, a);
  } else if (p.head_dim == 128) {
    hipLaunchKernelGGL((block_mass_kernel<128, 4>), grid, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((block_mass_kernel<64, 4>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_selection_quality(const Problem& p, const int32_t* rows, int32_t n_rows, const float* mass,
                                    const float* sel_mass, const float* scores, const int32_t* sel, int64_t ld,
                                    float* quality, hipStream_t stream) {
  int hkv_shift = 0;
  while ((1 << hkv_shift) < p.hkv) ++hkv_shift;
  if (n_rows == 0) return hipSuccess;
  QualityArgs a{p, rows, n_rows, mass, sel_mass, scores, sel, ld, quality, hkv_shift};
  const int64_t waves = (int64_t)n_rows << hkv_shift;
  hipLaunchKernelGGL(selection_quality_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace msa
