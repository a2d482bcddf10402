// attn_decode.hip — Main Branch of MSA for decode: one new query per
// sequence attends to the tokens of its (at most 16) selected blocks.
//
// Source: "MiniMax 模型迭代与竞品分析：从 Text-01、M1、M2 到 M3", §2: the
// softmax-attention equation and MSA step 4 (exact softmax over the chosen
// blocks only, at most 2048 tokens).  "前沿架构解码手记（三）" §2.1: with the
// block-major cache, each chosen block of one KV head is 128 rows of
// head_dim contiguous values, read whole.
//
// Decode moves ~1 MB of K/V per (sequence, group) at head_dim 128 for ~6
// MFLOP: it is bound by HBM bandwidth, so it uses plain vector ALU math and
// spreads the work over (slot, group, sequence) workgroups, each streaming
// one 128-token block of one KV head; a second pass merges the per-block
// partials of each head by log-sum-exp.
//   partial: scores of the group's heads against the block's keys (each
//            thread one key, half of head_dim), base-2 softmax statistics per
//            head, then P.V with each lane owning two output dims.
//   merge:   per (sequence, group), weights l_j * 2^(m_j - M) over the slots.
#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {

constexpr int kMaxGroup = 16;

struct DecodeArgs {
  Problem p;
  const uint16_t* q;
  const int32_t* sel;
  float* part_o;   // [num_seqs][hkv][16][G][D] normalised partial outputs
  float* part_st;  // [num_seqs][hkv][16][G][2] (max, sum) in base 2
  uint16_t* out;
};

size_t decode_workspace_bytes(const Problem& p) {
  const size_t parts = (size_t)p.num_seqs * p.hkv * kTopK * p.group;
  return ((parts * p.head_dim * sizeof(float) + 255) & ~(size_t)255) + parts * 2 * sizeof(float);
}

template <int D>
__global__ __launch_bounds__(256) void decode_partial_kernel(DecodeArgs a) {
  constexpr int DP = D / 2;            // output dim pairs
  constexpr int KG = 256 / DP;         // key groups in the P.V pass
  constexpr int KPG = kBlock / KG;     // keys per group
  __shared__ float q_s[kMaxGroup][D];
  __shared__ float s_s[kMaxGroup][kBlock];
  __shared__ float red_s[KG][kMaxGroup][D];
  __shared__ float stat_s[kMaxGroup][2];
  const Problem& p = a.p;
  const int slot = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int G = p.group;
  const int tid = threadIdx.x;
  const int r = p.cu_q[s];
  const int t = p.seq_lens[s] - 1;
  const int c = t >> 7;
  const int64_t part = (((int64_t)s * p.hkv + g) * kTopK + slot) * G;
  const int b = a.sel[((int64_t)r * p.hkv + g) * kTopK + slot];
  const int phys = (b >= 0 && b <= c) ? p.block_table[(int64_t)s * p.max_blocks_per_seq + b] : -1;
  if (phys < 0 || phys >= p.num_blocks) {
    if (tid < G) {
      a.part_st[(part + tid) * 2 + 0] = -__builtin_inff();
      a.part_st[(part + tid) * 2 + 1] = 0.f;
    }
    return;
  }
  const int nvalid = (b == c) ? (t & (kBlock - 1)) + 1 : kBlock;
  const int64_t key_stride = (int64_t)p.hkv * D;
  const uint16_t* kb = p.k + ((int64_t)phys * kBlock * p.hkv + g) * D;
  const uint16_t* vb = p.v + ((int64_t)phys * kBlock * p.hkv + g) * D;

  // V loads first, so they are in flight during the score pass.
  const int dp = tid % DP, kgrp = tid / DP;
  uint32_t vreg[KPG];
#pragma unroll
  for (int i = 0; i < KPG; ++i) {
    const int key = kgrp * KPG + i;
    vreg[i] = key < nvalid ? *reinterpret_cast<const uint32_t*>(vb + key * key_stride + dp * 2) : 0u;
  }
  // Query heads of the group, as float.
  for (int idx = tid; idx < G * D; idx += 256) {
    const int j = idx / D, d = idx - j * D;
    q_s[j][d] = bf16_to_f32(a.q[((int64_t)r * p.hq + g * G + j) * D + d]);
  }
  // Score pass: thread = (key, half of head_dim).
  const int key = tid >> 1, hd = tid & 1;
  u32x4 kreg[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i)
    kreg[i] = key < nvalid ? load16(kb + key * key_stride + hd * (D / 2) + i * 8) : u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  float acc[kMaxGroup];
#pragma unroll
  for (int j = 0; j < kMaxGroup; ++j) acc[j] = 0.f;
#pragma unroll
  for (int i = 0; i < D / 16; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float kv = bf16_to_f32((kreg[i][e >> 1] >> ((e & 1) * 16)) & 0xffffu);
      const int d = hd * (D / 2) + i * 8 + e;
#pragma unroll
      for (int j = 0; j < kMaxGroup; ++j)
        if (j < G) acc[j] += q_s[j][d] * kv;
    }
#pragma unroll
  for (int j = 0; j < kMaxGroup; ++j) {
    if (j < G) {
      const float tot = acc[j] + __shfl_xor(acc[j], 1);
      if (hd == 0) s_s[j][key] = key < nvalid ? tot * p.scale_log2e : -__builtin_inff();
    }
  }
  __syncthreads();
  // Softmax statistics: wave w handles heads w, w+4, ...; lane covers 2 keys.
  const int lane = tid & 63, wave = tid >> 6;
  for (int j = wave; j < G; j += 4) {
    const float z0 = s_s[j][lane], z1 = s_s[j][lane + 64];
    float m = fmaxf(z0, z1);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    const float e0 = fast_exp2(z0 - m), e1 = fast_exp2(z1 - m);
    s_s[j][lane] = e0;
    s_s[j][lane + 64] = e1;
    float l = e0 + e1;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
    if (lane == 0) {
      stat_s[j][0] = m;
      stat_s[j][1] = l;
    }
  }
  __syncthreads();
  // P.V: each thread two output dims for its key group, all heads.
  float o0[kMaxGroup], o1[kMaxGroup];
#pragma unroll
  for (int j = 0; j < kMaxGroup; ++j) o0[j] = o1[j] = 0.f;
#pragma unroll
  for (int i = 0; i < KPG; ++i) {
    const int kk = kgrp * KPG + i;
    const float v0 = bf16_to_f32(vreg[i] & 0xffffu), v1 = bf16_to_f32(vreg[i] >> 16);
#pragma unroll
    for (int j = 0; j < kMaxGroup; ++j)
      if (j < G) {
        const float pj = s_s[j][kk];
        o0[j] += pj * v0;
        o1[j] += pj * v1;
      }
  }
#pragma unroll
  for (int j = 0; j < kMaxGroup; ++j)
    if (j < G) {
      red_s[kgrp][j][dp * 2] = o0[j];
      red_s[kgrp][j][dp * 2 + 1] = o1[j];
    }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 256) {
    const int j = idx / D, d = idx - j * D;
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < KG; ++k) sum += red_s[k][j][d];
    a.part_o[(part + j) * D + d] = sum / stat_s[j][1];
  }
  if (tid < G) {
    a.part_st[(part + tid) * 2 + 0] = stat_s[tid][0];
    a.part_st[(part + tid) * 2 + 1] = stat_s[tid][1];
  }
}

template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  const Problem& p = a.p;
  const int g = blockIdx.x, s = blockIdx.y;
  const int G = p.group;
  const int r = p.cu_q[s];
  const int64_t part0 = ((int64_t)s * p.hkv + g) * kTopK * G;
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int j = idx / D, d = idx - j * D;
    float M = -__builtin_inff();
    for (int k = 0; k < kTopK; ++k) M = fmaxf(M, a.part_st[(part0 + k * G + j) * 2]);
    float L = 0.f, o = 0.f;
    for (int k = 0; k < kTopK; ++k) {
      const float l = a.part_st[(part0 + k * G + j) * 2 + 1];
      if (l <= 0.f) continue;
      const float w = l * fast_exp2(a.part_st[(part0 + k * G + j) * 2] - M);
      L += w;
      o += w * a.part_o[(part0 + k * G + j) * D + d];
    }
    a.out[((int64_t)r * p.hq + g * G + j) * D + d] = (uint16_t)f32_to_bf16_bits(o / L);
  }
}

hipError_t launch_attn_decode(const Problem& p, const uint16_t* q, const int32_t* sel, uint16_t* out, void* ws,
                              hipStream_t stream) {
  if (p.num_seqs == 0) return hipSuccess;
  const size_t parts = (size_t)p.num_seqs * p.hkv * kTopK * p.group;
  char* base = static_cast<char*>(ws);
  DecodeArgs a{p, q, sel, reinterpret_cast<float*>(base),
               reinterpret_cast<float*>(base + ((parts * p.head_dim * sizeof(float) + 255) & ~(size_t)255)), out};
  const dim3 pgrid(kTopK, p.hkv, p.num_seqs), mgrid(p.hkv, p.num_seqs);
  if (p.head_dim == 128) {
    hipLaunchKernelGGL(decode_partial_kernel<128>, pgrid, dim3(256), 0, stream, a);
    hipLaunchKernelGGL(decode_merge_kernel<128>, mgrid, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(decode_partial_kernel<64>, pgrid, dim3(256), 0, stream, a);
    hipLaunchKernelGGL(decode_merge_kernel<64>, mgrid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace msa
