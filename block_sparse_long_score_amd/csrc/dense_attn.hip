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

// One staged block: K and V of 128 keys, row-major [key][D], in 16-byte
// chunks placed at a per-row XOR of their index so that the operand reads
// touch every bank once per pass:
//   K (read as 16-byte rows of 16 keys x one chunk): slot = c ^ ((r/RPB) & (CPR-1));
//   V (read transposed, 4 keys x 4 chunks per 32 lanes): slot = c ^ (((r/RPB) & (CPR/4-1)) << 2),
// with CPR chunks per row and RPB rows per 256 bytes of banks.  For the rows
// a lane reads, both XOR terms depend on the lane only, so every operand
// address is a per-lane base plus a compile-time offset.
template <int D>
struct DenseBuf {
  uint16_t k[kBlock * D];
  uint16_t v[kBlock * D];
};

template <int D>
__device__ __forceinline__ int dense_kslot(int r, int c) {
  constexpr int CPR = D / 8, RPB = 128 / D;
  return c ^ ((r / RPB) & (CPR - 1));
}

template <int D>
__device__ __forceinline__ int dense_vslot(int r, int c) {
  constexpr int CPR = D / 8, RPB = 128 / D;
  return c ^ (((r / RPB) & (CPR / 4 - 1)) << 2);
}

// Per-lane byte offsets of the block copy: round i moves slots
// (8i + wave) * 64 + lane of K and of V (row r = slot / CPR), reading the
// global chunk that belongs in that slot.
template <int D>
struct DmaLane {
  static constexpr int CPR = D / 8;
  static constexpr int ROUNDS = kBlock * CPR / (64 * kDenseWaves);
  uint32_t koff[ROUNDS], voff[ROUNDS];  // bytes from the block's first key row
  int row[ROUNDS];
};

template <int D>
__device__ __forceinline__ DmaLane<D> dma_lane(int wave, int lane, int64_t key_stride) {
  DmaLane<D> d;
#pragma unroll
  for (int i = 0; i < DmaLane<D>::ROUNDS; ++i) {
    const int slot_idx = (i * kDenseWaves + wave) * 64 + lane;
    const int r = slot_idx / DmaLane<D>::CPR, sl = slot_idx % DmaLane<D>::CPR;
    d.row[i] = r;
    d.koff[i] = (uint32_t)((r * key_stride + dense_kslot<D>(r, sl) * 8) * 2);
    d.voff[i] = (uint32_t)((r * key_stride + dense_vslot<D>(r, sl) * 8) * 2);
  }
  return d;
}

// Asynchronous copy of one block of group g into LDS with the global->LDS
// loads (each wave instruction fills 64 consecutive 16-byte slots).  In a
// block cut short by the end of the sequence, keys at or after `valid` read
// the last valid key instead: finite data, and always masked since they lie
// after every query position.
template <int D>
__device__ __forceinline__ void dense_dma(DenseBuf<D>& B, const DmaLane<D>& dl, int wave, const uint16_t* kg,
                                          const uint16_t* vg, int64_t key_stride, int valid) {
  const char* kb = reinterpret_cast<const char*>(kg);
  const char* vb = reinterpret_cast<const char*>(vg);
  const bool full = valid == kBlock;
#pragma unroll
  for (int i = 0; i < DmaLane<D>::ROUNDS; ++i) {
    const int run = i * kDenseWaves + wave;
    uint32_t ko = dl.koff[i], vo = dl.voff[i];
    if (!full && dl.row[i] >= valid) {
      const uint32_t shift = (uint32_t)((dl.row[i] - (valid - 1)) * key_stride * 2);
      ko -= shift;
      vo -= shift;
    }
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(kb + ko),
                                     reinterpret_cast<__attribute__((address_space(3))) void*>(
                                         reinterpret_cast<uintptr_t>(&B.k[run * 512])),
                                     16, 0, 0);
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(vb + vo),
                                     reinterpret_cast<__attribute__((address_space(3))) void*>(
                                         reinterpret_cast<uintptr_t>(&B.v[run * 512])),
                                     16, 0, 0);
  }
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Transposed LDS read (gfx950 ds_read_b64_tr_b16): within each group of 16
// lanes, lane 4a+b receives element b of the 4-element row addressed by
// lane 4j+a, for j = 0..3.
typedef __attribute__((address_space(3))) const char lds_byte;

__device__ __forceinline__ i16x4 lds_read_tr16(lds_byte* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

// Per-lane byte offsets of the operand reads within a staged block.
//   K, k-step ks: row l32 (+ 32 t4), chunk 2ks + half.
//   V^T, dim tile n: lane (group gi = lane/16, s = lane%16 = 4j + a) addresses
//   row 4(gi/2) + j (+ 16kk + 8q), dims 32n + 16(gi%2) + 4a .. +3, so the
//   transposed read hands lane (d = 32n + lane%32, half) keys
//   16kk + 4half + 8q + {0..3}: the key order of the P^T operand.
template <int D>
struct OpLane {
  uint32_t k[D / 16];
  uint32_t v[D / 32];
};

template <int D>
__device__ __forceinline__ OpLane<D> op_lane(int lane) {
  OpLane<D> o;
  const int half = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) o.k[ks] = (uint32_t)((l32 * D + dense_kslot<D>(l32, 2 * ks + half) * 8) * 2);
  const int gi = lane >> 4, s16 = lane & 15;
  const int jr = s16 >> 2, a4 = s16 & 3;
  const int r = 4 * (gi >> 1) + jr;
#pragma unroll
  for (int n = 0; n < D / 32; ++n) {
    const int c = 4 * n + 2 * (gi & 1) + (a4 >> 1);
    o.v[n] = (uint32_t)((r * D + dense_vslot<D>(r, c) * 8 + (a4 & 1) * 4) * 2);
  }
  return o;
}

// One block for this wave's 32 rows: S^T = K Q^T, mask, online softmax, O^T += V^T P^T.
template <int D>
__device__ __forceinline__ void dense_block(const DenseBuf<D>& B, const OpLane<D>& ol, const bf16x8 (&bq)[D / 16],
                                           f32x16 (&oacc)[D / 32], float& m, float& l, float c, bool masked,
                                           int lim) {
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const char* kb = reinterpret_cast<const char*>(B.k);
  lds_byte* vb = (lds_byte*)(B.v);
  f32x16 sacc[4];
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4)
    sacc[t4] = f32x16{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const bf16x8 ak = as_bf16x8(*reinterpret_cast<const u32x4*>(kb + ol.k[ks] + t4 * 32 * D * 2));
      sacc[t4] = mfma32(ak, bq[ks], sacc[t4]);
    }
  __builtin_amdgcn_sched_barrier(0);
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
  bf16x8 pb[8];
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
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
#pragma unroll
    for (int n = 0; n < D / 32; ++n) {
      const i16x4 lo = lds_read_tr16(vb + ol.v[n] + (16 * kk) * D * 2);
      const i16x4 hi = lds_read_tr16(vb + ol.v[n] + (16 * kk + 8) * D * 2);
      const u32x2 lw = __builtin_bit_cast(u32x2, lo), hw = __builtin_bit_cast(u32x2, hi);
      oacc[n] = mfma32(as_bf16x8(u32x4{lw[0], lw[1], hw[0], hw[1]}), pb[kk], oacc[n]);
    }
}

template <int D>
__global__ __launch_bounds__(64 * kDenseWaves, 2) void dense_prefill_kernel(DenseArgs a) {
  __shared__ DenseBuf<D> buf0, buf1;
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
  const DmaLane<D> dl = dma_lane<D>(wave, lane, key_stride);
  const OpLane<D> ol = op_lane<D>(lane);

  // Block b is staged in buf0 (b even) or buf1 (b odd), one block ahead:
  // the copy of b+1 runs while block b is computed.  Blocks whose table
  // entry is out of range hold no keys: neither copied nor computed.  The
  // table entries of blocks b+2 and b+3 are loaded by alternate lanes while
  // block b is computed and read out of lanes 0 and 1 after the next
  // barrier, so no wait for them ever waits for a copy in flight.
  auto phys_ok = [&](int b, int ph) { return (b < nb && ph >= 0 && ph < p.num_blocks) ? ph : -1; };
  auto stage = [&](DenseBuf<D>& B, int b, int phys) {
    if (phys < 0) return;
    const int64_t base = ((int64_t)phys * kBlock * p.hkv + g) * D;
    dense_dma<D>(B, dl, wave, p.k + base, p.v + base, key_stride, min(kBlock, seq_len - b * kBlock));
  };
  auto run = [&](const DenseBuf<D>& B, int b, int phys) {
    if (b > last_b || phys < 0) return;
    dense_block<D>(B, ol, bq, oacc, m, l, c, b >= first_masked, t - b * kBlock);
  };
  int pair = bt[min(lane & 1, nb - 1)];
  int ph_cur = phys_ok(0, __builtin_amdgcn_readlane(pair, 0));
  int ph_nxt = phys_ok(1, __builtin_amdgcn_readlane(pair, 1));
  stage(buf0, 0, ph_cur);
  for (int b = 0; b < nb; b += 2) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of block b have landed
    __syncthreads();                // everyone's have, and block b-1 (buf1) is no longer read
    pair = bt[min(b + 2 + (lane & 1), nb - 1)];
    stage(buf1, b + 1, ph_nxt);
    run(buf0, b, ph_cur);
    if (b + 1 >= nb) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int ph_odd = ph_nxt;
    ph_cur = phys_ok(b + 2, __builtin_amdgcn_readlane(pair, 0));
    ph_nxt = phys_ok(b + 3, __builtin_amdgcn_readlane(pair, 1));
    stage(buf0, b + 2, ph_cur);
    run(buf1, b + 1, ph_odd);
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
    hipLaunchKernelGGL(dense_prefill_kernel<128>, grid, dim3(64 * kDenseWaves), 0, stream, a);
  else
    hipLaunchKernelGGL(dense_prefill_kernel<64>, grid, dim3(64 * kDenseWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace msa
