// dense_attn.hip — dense causal GQA softmax attention over the block-major
// KV cache: every query row attends to all keys at or before its position.
//
// Source: "MiniMax 模型迭代与竞品分析：从 Text-01、M1、M2 到 M3", §2: the
// softmax-attention equation (scores q.k/sqrt(d_k), causal, softmax over the
// attended keys, probability-weighted sum of values) and, in §2-§3, the
// layers and the training warmup that run full attention beside the sparse
// ones.  It is MSA with every causal block selected, on the cache MSA uses.
//
// Schedule (queries outer).  One workgroup of 8 waves per (sequence, tile of
// 256 query rows, query head); wave w owns 32 consecutive rows, two waves
// share each SIMD.  The workgroup walks the causal blocks in order.  K and V
// of a block are copied from the cache straight into LDS with the
// asynchronous global->LDS loads (row-major, 16-byte chunks XOR-swizzled per
// row), double-buffered so the copies of the next block overlap the math of
// this one.  Every wave runs its rows against the staged block on the
// 32x32x16 bf16 MFMA: S^T = K Q^T with K rows as the A operand, then
// O^T += V^T P^T with the V^T operand read by the LDS transpose load
// (ds_read_b64_tr_b16), so nothing is transposed by the vector ALU.  The
// softmax is online, in base 2; only the one or two blocks that hold the
// tile's own positions are masked.  The running maximum is raised only when
// a block's maximum exceeds it by more than 2^8, so the accumulators are
// rescaled rarely; numerator and denominator share the reference value, so
// the result is unchanged.  Per wave and block the operand reads move 64 KB
// out of LDS for 64 MFMAs (32 query rows per wave), which bounds the kernel
// at roughly half of the MFMA peak on this LDS.
//
// Work order.  Workgroups are dispatched round-robin over the 8 XCDs
// (workgroup i runs on XCD i % 8), each with its own L2.  The mapping from
// workgroup id to (tile, sequence, head) puts all heads of one KV group, for
// the same tiles, on the same XCD, so they read the group's K/V blocks from
// that XCD's L2 at about the same time; tiles run latest positions first
// (the longest rows first) for load balance.
#include "attn_tiles.h"
#include "msa_kernels.h"

#include <type_traits>

namespace msa {

constexpr int kDenseRows = 256;   // query rows of one head per workgroup
constexpr int kDenseWaves = 8;    // 32 rows each; two waves per SIMD

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

// Mask (keys after the row's position, in the blocks that hold the tile's
// own positions), online softmax update and P rounded to bf16 in the key
// order of the P^T operand.  The running maximum is raised only when the
// block's maximum exceeds it by more than 8 (log2 units), so the O
// accumulators are rescaled rarely.
template <int D>
__device__ __forceinline__ void dense_softmax(f32x16 (&sacc)[4], bool masked, int lim, float c, float& m, float& l,
                                             f32x16 (&oacc)[D / 32], bf16x8 (&pb)[8]) {
  __builtin_amdgcn_sched_barrier(0);
  const int half = (threadIdx.x >> 5) & 1;
  if (masked) {
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
  for (int kk = 0; kk < 8; ++kk) {
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      e[i] = fast_exp2(fmaf(sacc[kk >> 1][(kk & 1) * 8 + i], c, -m));
      sum += e[i];
    }
    pb[kk] = as_bf16x8(u32x4{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                             pack_bf16x2(e[6], e[7])});
  }
  l += sum + swap_halves(sum);
}

template <int D>
__global__ __launch_bounds__(64 * kDenseWaves, 2) void dense_prefill_kernel(DenseArgs a) {
  __shared__ uint16_t k0[kBlock * D], k1[kBlock * D], v0[kBlock * D], v1[kBlock * D];
  const Problem& p = a.p;
  int tf, s, h;
  if (!dense_item(a, tf, s, h)) return;
  const int q_beg = p.cu_q[s], q_end = p.cu_q[s + 1];
  const int r_hi = q_end - kDenseRows * tf;  // rows [r_hi - 256, r_hi) of which those >= q_beg exist
  if (r_hi <= q_beg) return;
  const int g = h / p.group;
  const int seq_len = p.seq_lens[s];
  const int nb = ((seq_len - 1 - kDenseRows * tf) >> 7) + 1;  // blocks up to the tile's last position
  const int32_t* bt = p.block_table + (int64_t)s * p.max_blocks_per_seq;
  const int64_t key_stride = (int64_t)p.hkv * D;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int row0 = r_hi - kDenseRows + 32 * wave;  // this wave's first (possibly absent) row
  const int my_row = max(row0 + l32, q_beg);       // rows before the sequence's queries stand in for its first
  const int t = seq_len - (q_end - my_row);        // this lane's query position
  const int t_first = seq_len - (q_end - max(row0, q_beg));
  const int t_last = seq_len - (q_end - (row0 + 31));
  const bool active = row0 + 31 >= q_beg;          // wave has rows of its own
  const int last_b = active ? t_last >> 7 : -1;
  const int first_masked = t_first >> 7;
  const bool lead = wave < kDenseWaves / 2;        // waves 0-3 lead, 4-7 trail (one of each per SIMD)

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
  f32x16 sacc[4];
  bf16x8 pb[8];
  const DmaLane<D, kDenseWaves> dl = dma_lane<D, kDenseWaves>(wave, lane, key_stride);
  const OpLane<D> ol = op_lane<D>(lane);

  // Ping-pong schedule.  Barrier interval i computes, per wave, the matrix
  // products P.V of block i-1 and S = K.Q of block i, and one softmax:
  // leading waves run the products first and then the softmax of block i,
  // trailing waves run the softmax of block i-1 first and then the
  // products.  The two waves that share a SIMD thus alternate between the
  // matrix cores and the vector ALU.  Interval i reads K_i and V_{i-1};
  // meanwhile K_{i+1} and V_i are copied into the other K and V buffers.
  // Blocks whose table entry is out of range hold no keys: neither copied
  // nor computed.  Table entries are loaded two intervals ahead by alternate
  // lanes and read out of lane 0 after the next barrier.
  auto phys_ok = [&](int b, int ph) { return (b >= 0 && b < nb && ph >= 0 && ph < p.num_blocks) ? ph : -1; };
  auto computes = [&](int b, int ph) { return b >= 0 && b <= last_b && ph >= 0; };
  auto block_src = [&](int ph) { return ((int64_t)ph * kBlock * p.hkv + g) * D; };
  auto valid_of = [&](int b) { return min(kBlock, seq_len - b * kBlock); };

  int pair = bt[min(lane & 1, nb - 1)];
  int ph_prev = -1;
  int ph_cur = phys_ok(0, __builtin_amdgcn_readlane(pair, 0));
  int ph_next = phys_ok(1, __builtin_amdgcn_readlane(pair, 1));
  if (ph_cur >= 0) block_dma<D, kDenseWaves, false>(k0, dl, wave, p.k + block_src(ph_cur), key_stride, valid_of(0));

  auto interval = [&](auto parity, int i) {
    constexpr int P = decltype(parity)::value;
    uint16_t* knext = P ? k0 : k1;
    uint16_t* vcur = P ? v1 : v0;
    lds_byte* kcur = opaque_lds(P ? k1 : k0);
    lds_byte* vprev = opaque_lds(P ? v0 : v1);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies for this interval have landed
    __syncthreads();                // everyone's have, and the previous interval's buffers are free
    if (i >= 1) ph_next = phys_ok(i + 1, __builtin_amdgcn_readlane(pair, 0));
    pair = bt[min(i + 2 + (lane & 1), nb - 1)];
    if (ph_next >= 0)
      block_dma<D, kDenseWaves, false>(knext, dl, wave, p.k + block_src(ph_next), key_stride, valid_of(i + 1));
    if (i < nb && ph_cur >= 0)
      block_dma<D, kDenseWaves, true>(vcur, dl, wave, p.v + block_src(ph_cur), key_stride, valid_of(i));
    const bool pv = computes(i - 1, ph_prev), sc = i < nb && computes(i, ph_cur);
    // leading: P.V(i-1), S(i), softmax(i); trailing: softmax(i-1), P.V(i-1), S(i)
    if (!lead && pv) dense_softmax<D>(sacc, i - 1 >= first_masked, t - (i - 1) * kBlock, c, m, l, oacc, pb);
    if (pv) tile_pv<D, true>(vprev, ol, pb, oacc);
    if (sc) {
      tile_scores<D>(kcur, ol, bq, sacc);
    } else {  // defined on every path: no S value is live across the P.V products
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
        sacc[t4] = f32x16{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    }
    if (lead && sc) dense_softmax<D>(sacc, i >= first_masked, t - i * kBlock, c, m, l, oacc, pb);
    ph_prev = ph_cur;
    ph_cur = ph_next;
    ph_next = -1;
  };
  for (int i = 0; i <= nb; i += 2) {
    interval(std::integral_constant<int, 0>(), i);
    if (i + 1 > nb) break;
    interval(std::integral_constant<int, 1>(), i + 1);
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

// ------------------------------------------------------------------ decode

// Dense decode: one query row per sequence attends to its whole context.
// Schedule: one 16-wave workgroup per (sequence, group, split of 64 blocks);
// the waves take the split's blocks in turn (wave w: blocks w, w+16, ...),
// each keeping a running softmax over its blocks (DecodeWave: scores on the
// 16x16x32 MFMA with the group's heads on N, P.V on the vector ALU), and
// combine in LDS into the split's normalised output and log2 mass.  A merge
// pass combines the splits.  HBM-bound: every K and V row of the context is
// read once per (sequence, group).
constexpr int kDecodeWaves = 16;
constexpr int kDecodeSplit = 64;  // blocks per workgroup

struct DenseDecodeArgs {
  Problem p;
  const uint16_t* q;
  float* part_o;    // [num_seqs][hkv][n_split][G][D]: the split's normalised output
  float* part_lse;  // [num_seqs][hkv][n_split][G]: log2 of the split's softmax mass, in the units of the scores
  uint16_t* out;
  int n_split;
};

template <int D, int GM>
__global__ __launch_bounds__(64 * kDecodeWaves) void dense_decode_kernel(DenseDecodeArgs a) {
  using W = DecodeWave<D, GM>;
  __shared__ float p_s[kDecodeWaves][GM][W::SUB];
  __shared__ float alpha_s[kDecodeWaves][GM];
  __shared__ float m_s[kDecodeWaves][GM], l_s[kDecodeWaves][GM];
  __shared__ __attribute__((aligned(16))) float o_s[kDecodeWaves][GM][D];
  // Each wave's K staging: inside its own o_s rows when they are large
  // enough (they are written only after the wave's last block), else apart.
  constexpr bool kStageInOut = GM * D * 4 >= W::STAGE * 2;
  __shared__ __attribute__((aligned(16))) uint16_t kst_s[kStageInOut ? 1 : kDecodeWaves][kStageInOut ? 1 : W::STAGE];
  const Problem& p = a.p;
  const int G = p.group;
  const int split = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int t = p.seq_lens[s] - 1;
  const int nb = (t >> 7) + 1;
  const int b0 = split * kDecodeSplit;
  if (b0 >= nb) return;
  const int r = p.cu_q[s];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t* bt = p.block_table + (int64_t)s * p.max_blocks_per_seq;
  W st;
  {
    bf16x8 bq[W::KS];
    st.load_q(a.q + ((int64_t)r * p.hq + g * G) * D, G, bq);
    const int b_end = min(b0 + kDecodeSplit, nb);
    for (int b = b0 + w; b < b_end; b += kDecodeWaves) {
      const int phys = bt[b];
      if (phys < 0 || phys >= p.num_blocks) continue;  // absent blocks hold no keys
      uint16_t* stage = kStageInOut ? reinterpret_cast<uint16_t*>(&o_s[w][0][0]) : &kst_s[kStageInOut ? 0 : w][0];
      st.template attend_block<false>(p.k, p.v, ((int64_t)phys * kBlock * p.hkv + g) * D, (int64_t)p.hkv * D,
                                      min(kBlock, t - b * kBlock + 1), bq, p.scale_log2e, p_s[w], alpha_s[w], stage);
    }
  }
  st.store(o_s[w], m_s[w], l_s[w]);
  __syncthreads();
  const int64_t part = (((int64_t)s * p.hkv + g) * a.n_split + split) * G;
  for (int idx = threadIdx.x; idx < G * (D / 2); idx += blockDim.x) {
    const int j = idx / (D / 2), d = (idx - j * (D / 2)) * 2;
    float o0, o1, L, M;
    combine_waves<D, GM, kDecodeWaves>(o_s, m_s, l_s, j, d, o0, o1, L, M);
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    *reinterpret_cast<f32x2*>(a.part_o + (part + j) * D + d) = f32x2{o0 * inv, o1 * inv};
    if (d == 0) a.part_lse[part + j] = L > 0.f ? M + __log2f(L) : -__builtin_inff();
  }
}

// Merge of the splits: per (sequence, head, dim pair) a log-sum-exp over the
// sequence's splits, rounded to bf16.
template <int D>
__global__ __launch_bounds__(256) void dense_decode_merge_kernel(DenseDecodeArgs a) {
  const Problem& p = a.p;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_seq = (int64_t)p.hq * (D / 2);
  if (idx >= per_seq * p.num_seqs) return;
  const int s = (int)(idx / per_seq);
  const int rem = (int)(idx - s * per_seq);
  const int h = rem / (D / 2), d = (rem - h * (D / 2)) * 2;
  const int G = p.group;
  const int g = h / G, j = h - g * G;
  const int nb = ((p.seq_lens[s] - 1) >> 7) + 1;
  const int nsp = (nb + kDecodeSplit - 1) / kDecodeSplit;
  const int64_t part0 = ((int64_t)s * p.hkv + g) * a.n_split * G + j;
  float M = -__builtin_inff();
  for (int sp = 0; sp < nsp; ++sp) M = fmaxf(M, a.part_lse[part0 + (int64_t)sp * G]);
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  for (int sp = 0; sp < nsp; ++sp) {
    const float lse = a.part_lse[part0 + (int64_t)sp * G];
    const float f = lse > -__builtin_inff() ? fast_exp2(lse - M) : 0.f;
    const f32x2 o = *reinterpret_cast<const f32x2*>(a.part_o + (part0 + (int64_t)sp * G) * D + d);
    L += f;
    o0 = fmaf(f, o[0], o0);
    o1 = fmaf(f, o[1], o1);
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  *reinterpret_cast<uint32_t*>(a.out + ((int64_t)p.cu_q[s] * p.hq + h) * D + d) = pack_bf16x2(o0 * inv, o1 * inv);
}

static int decode_splits(const Problem& p, int max_ctx_blocks) {
  return std::max(1, (max_ctx_blocks + kDecodeSplit - 1) / kDecodeSplit);
}

size_t dense_decode_workspace_bytes(const Problem& p, int max_ctx_blocks) {
  const int64_t parts = (int64_t)p.num_seqs * p.hkv * decode_splits(p, max_ctx_blocks) * p.group;
  const size_t o = ((sizeof(float) * parts * p.head_dim) + 255) & ~(size_t)255;
  return o + sizeof(float) * parts;
}

template <int D>
static void launch_dense_decode_t(const DenseDecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.n_split, a.p.hkv, a.p.num_seqs);
  if (a.p.group <= 4)
    hipLaunchKernelGGL((dense_decode_kernel<D, 4>), grid, dim3(64 * kDecodeWaves), 0, stream, a);
  else if (a.p.group <= 6)
    hipLaunchKernelGGL((dense_decode_kernel<D, 6>), grid, dim3(64 * kDecodeWaves), 0, stream, a);
  else if (a.p.group <= 8)
    hipLaunchKernelGGL((dense_decode_kernel<D, 8>), grid, dim3(64 * kDecodeWaves), 0, stream, a);
  else
    hipLaunchKernelGGL((dense_decode_kernel<D, 16>), grid, dim3(64 * kDecodeWaves), 0, stream, a);
  const int64_t threads = (int64_t)a.p.num_seqs * a.p.hq * (D / 2);
  hipLaunchKernelGGL(dense_decode_merge_kernel<D>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a);
}

hipError_t launch_dense_decode(const Problem& p, const uint16_t* q, uint16_t* out, void* ws, int max_ctx_blocks,
                               hipStream_t stream) {
  if (p.total_q == 0) return hipSuccess;
  const int n_split = decode_splits(p, max_ctx_blocks);
  const int64_t parts = (int64_t)p.num_seqs * p.hkv * n_split * p.group;
  char* base = static_cast<char*>(ws);
  const size_t o_bytes = ((sizeof(float) * parts * p.head_dim) + 255) & ~(size_t)255;
  const DenseDecodeArgs a{p, q, reinterpret_cast<float*>(base), reinterpret_cast<float*>(base + o_bytes), out, n_split};
  if (p.head_dim == 128)
    launch_dense_decode_t<128>(a, stream);
  else
    launch_dense_decode_t<64>(a, stream);
  return hipGetLastError();
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
    hipLaunchKernelGGL(dense_prefill_kernel<128>, grid, dim3(64 * kDenseWaves), 0, stream, a);
  else
    hipLaunchKernelGGL(dense_prefill_kernel<64>, grid, dim3(64 * kDenseWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace msa
