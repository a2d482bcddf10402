// attn_prefill.hip — Main Branch of MSA for prefill: exact softmax attention
// of every query row over the tokens of its selected blocks.
//
// Source: "MiniMax 模型迭代与竞品分析：从 Text-01、M1、M2 到 M3", §2: the
// softmax-attention equation (scores q.k/sqrt(d_k), softmax over the attended
// keys, probability-weighted sum of values) and MSA step 4 (standard softmax
// attention restricted to the chosen blocks, at most 16 x 128 = 2048 tokens).
// "MiniMax：Text-01 / M1 → M2.7 → M3", §5 names a KV-outer kernel design for
// the block-level irregular access; "前沿架构解码手记（三）" §2.1 motivates the
// block-major cache: a chosen block is one contiguous piece per head.
//
// Schedule (blocks outer).  Every (query, group) row selects up to 15
// non-local blocks at random-looking positions, so queries that share a block
// are scattered: loading the selected blocks per query would move 1 MB of K/V
// per (query, group) at head_dim 128.  Instead:
//   1. invert the selections into one list of (query row, slot) entries per
//      (physical block, group) — a counting sort: count, scan, fill;
//   2. kvouter: one workgroup per chunk of a list stages the block's K and V
//      (one group) in LDS once and runs every listed query's heads against it
//      with bf16 MFMA, writing a partial result per (row, slot, head): the
//      block-local softmax statistics (max, sum) and the normalised output,
//      stored as fp16 scaled by a power of two;
//   3. merge_local: per tile of queries of one block, attend to the local
//      (causal) block directly and fold in the partials of the other selected
//      blocks by log-sum-exp, then round the result to bf16.
// The softmax works in base 2 with the scale folded into log2(e).
//
// MFMA mapping (32x32x16 bf16, wave64), per tile of 32 (query, head) rows:
//   S^T[128 keys x 32 rows] = K[keys x D] * Q^T[D x rows]   (K from LDS, Q from HBM)
//   O^T[D x 32 rows]        = V^T[D x keys] * P^T[keys x rows]
// With keys on the M axis each lane owns one row, so row max/sum are in-lane
// plus one exchange between wave halves, and the S^T accumulators, rounded to
// bf16, are directly the B operand of the P.V product; V is stored transposed
// in LDS so its A operand is two 8-byte reads.
#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {

constexpr int kSlots = kTopK - 1;  // non-local blocks per row

// ---------------------------------------------------------------- workspace

struct PrefillWs {
  size_t cnt, off, coff, cursor, chunk_list, entries, part_o, part_st, total;
  int64_t n_lists, max_entries, max_chunks;
  int chunk;  // entries per kvouter workgroup
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int prefill_chunk(const Problem& p) {
  int ch = 384 / p.group;  // about 12 row tiles of 32 per workgroup
  return ch < 8 ? 8 : ch;
}

static PrefillWs prefill_layout(const Problem& p) {
  PrefillWs w{};
  w.chunk = prefill_chunk(p);
  w.n_lists = (int64_t)p.num_blocks * p.hkv;
  w.max_entries = (int64_t)p.total_q * p.hkv * kSlots;
  w.max_chunks = (w.max_entries + w.chunk - 1) / w.chunk + std::min<int64_t>(w.n_lists, w.max_entries);
  const int64_t parts = w.max_entries * p.group;
  size_t o = 0;
  w.cnt = o;        o = align256(o + sizeof(int32_t) * w.n_lists);
  w.off = o;        o = align256(o + sizeof(int32_t) * (w.n_lists + 1));
  w.coff = o;       o = align256(o + sizeof(int32_t) * (w.n_lists + 1));
  w.cursor = o;     o = align256(o + sizeof(int32_t) * w.n_lists);
  w.chunk_list = o; o = align256(o + sizeof(int32_t) * (w.max_chunks + 1));
  w.entries = o;    o = align256(o + sizeof(int32_t) * (w.max_entries + 1));
  w.part_o = o;     o = align256(o + sizeof(uint16_t) * parts * p.head_dim);
  w.part_st = o;    o = align256(o + sizeof(float) * 4 * parts);
  w.total = o;
  return w;
}

size_t prefill_workspace_bytes(const Problem& p) { return prefill_layout(p).total; }

// ------------------------------------------------------- selection inversion

struct CsrArgs {
  Problem p;
  const int32_t* sel;
  int32_t* cnt;
  int32_t* off;
  int32_t* coff;
  int32_t* cursor;
  int32_t* chunk_list;
  int32_t* entries;
  int64_t n_lists;
  int hkv_shift;
  int chunk;
};

__global__ __launch_bounds__(256) void csr_zero_kernel(int32_t* __restrict__ cnt, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    cnt[i] = 0;
}

// The list a (row, slot) entry belongs to, or -1 for empty/local slots.
__device__ __forceinline__ int64_t entry_list(const CsrArgs& a, int64_t idx) {
  const Problem& p = a.p;
  const int b = a.sel[idx];
  if (b < 0 || (idx & 15) >= kSlots) return -1;  // the local block is always the last of <= 16
  const int64_t R = idx >> 4;
  const int r = (int)(R >> a.hkv_shift);
  const int g = (int)(R & ((1 << a.hkv_shift) - 1));
  const int s = seq_of_row(p.cu_q, p.num_seqs, r);
  const int t = p.seq_lens[s] - (p.cu_q[s + 1] - r);
  if (b >= (t >> 7)) return -1;  // the local block is attended in merge_local
  const int phys = p.block_table[(int64_t)s * p.max_blocks_per_seq + b];
  if (phys < 0 || phys >= p.num_blocks) return -1;
  return ((int64_t)phys << a.hkv_shift) + g;
}

__global__ __launch_bounds__(256) void csr_count_kernel(CsrArgs a) {
  const int64_t n = ((int64_t)a.p.total_q << a.hkv_shift) * kTopK;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int64_t list = entry_list(a, idx);
  if (list >= 0) atomicAdd(a.cnt + list, 1);
}

// One workgroup: exclusive scans of the list sizes (entry offsets) and of the
// per-list chunk counts (chunk offsets); also clears the fill cursors.
__global__ __launch_bounds__(1024) void csr_scan_kernel(CsrArgs a) {
  __shared__ int64_t sums[2][1024];
  const int tid = threadIdx.x;
  const int64_t n = a.n_lists;
  const int64_t per = (n + 1023) / 1024;
  const int64_t lo = std::min<int64_t>(n, tid * per), hi = std::min<int64_t>(n, lo + per);
  int64_t se = 0, sc = 0;
  for (int64_t i = lo; i < hi; ++i) {
    const int c = a.cnt[i];
    se += c;
    sc += (c + a.chunk - 1) / a.chunk;
  }
  sums[0][tid] = se;
  sums[1][tid] = sc;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {  // inclusive Hillis-Steele scan
    int64_t ve = 0, vc = 0;
    if (tid >= d) { ve = sums[0][tid - d]; vc = sums[1][tid - d]; }
    __syncthreads();
    sums[0][tid] += ve;
    sums[1][tid] += vc;
    __syncthreads();
  }
  int64_t e = sums[0][tid] - se, c = sums[1][tid] - sc;
  for (int64_t i = lo; i < hi; ++i) {
    const int k = a.cnt[i];
    a.off[i] = (int32_t)e;
    a.coff[i] = (int32_t)c;
    a.cursor[i] = 0;
    e += k;
    c += (k + a.chunk - 1) / a.chunk;
  }
  if (tid == 1023) {
    a.off[n] = (int32_t)sums[0][1023];
    a.coff[n] = (int32_t)sums[1][1023];
  }
}

__global__ __launch_bounds__(256) void csr_fill_kernel(CsrArgs a) {
  const int64_t n = ((int64_t)a.p.total_q << a.hkv_shift) * kTopK;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int64_t list = entry_list(a, idx);
  if (list < 0) return;
  const int pos = a.off[list] + atomicAdd(a.cursor + list, 1);
  a.entries[pos] = (int32_t)idx;  // (R << 4) | slot
}

__global__ __launch_bounds__(256) void csr_chunk_map_kernel(CsrArgs a) {
  const int64_t list = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (list >= a.n_lists) return;
  for (int j = a.coff[list]; j < a.coff[list + 1]; ++j) a.chunk_list[j] = (int32_t)list;
}

// ------------------------------------------------------------ shared pieces

template <int D>
struct Lds {
  static constexpr int KP = D + 8;    // K row pitch (bf16): rows stay 16-byte aligned
  static constexpr int VP = 128 + 8;  // V^T row pitch (bf16)
  uint16_t k[128 * KP];
  uint16_t vt[D * VP];
};

// Stage one block of one KV head into LDS: K as [key][d], V as [d][key].
// Keys at or after `valid` are written as zeros (never read from the cache).
template <int D>
__device__ __forceinline__ void stage_block(Lds<D>& sm, const uint16_t* __restrict__ kg,
                                            const uint16_t* __restrict__ vg, int64_t key_stride, int valid) {
  constexpr int C8 = D / 8;
  for (int idx = threadIdx.x; idx < 128 * C8; idx += blockDim.x) {
    const int key = idx / C8, c8 = idx - key * C8;
    u32x4 v = key < valid ? load16(kg + key * key_stride + c8 * 8) : u32x4{0u, 0u, 0u, 0u};
    store16(&sm.k[key * Lds<D>::KP + c8 * 8], v);
  }
  for (int idx = threadIdx.x; idx < 32 * C8; idx += blockDim.x) {
    const int k4 = idx / C8, c8 = idx - k4 * C8;
    u32x4 r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = k4 * 4 + i;
      r[i] = key < valid ? load16(vg + key * key_stride + c8 * 8) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) * 16;
      const uint32_t x0 = (r[0][e >> 1] >> sh) & 0xffffu, x1 = (r[1][e >> 1] >> sh) & 0xffffu;
      const uint32_t x2 = (r[2][e >> 1] >> sh) & 0xffffu, x3 = (r[3][e >> 1] >> sh) & 0xffffu;
      *reinterpret_cast<u32x2*>(&sm.vt[(c8 * 8 + e) * Lds<D>::VP + k4 * 4]) = u32x2{x0 | (x1 << 16), x2 | (x3 << 16)};
    }
  }
}

// Scores of 32 rows against the staged block: S^T, 4 key tiles.
template <int D>
__device__ __forceinline__ void block_scores(const Lds<D>& sm, const bf16x8 (&bq)[D / 16], f32x16 (&sacc)[4]) {
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    __builtin_amdgcn_sched_barrier(0);  // one key tile at a time: bounds live operand registers
    sacc[m] = f32x16{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 ak = as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.k[(m * 32 + l32) * Lds<D>::KP + ks * 16 + half * 8]));
      sacc[m] = mfma32(ak, bq[ks], sacc[m]);
    }
  }
}

// O^T = V^T P^T for 32 rows; P given by the (exponentiated) S^T accumulators.
template <int D>
__device__ __forceinline__ void block_pv(const Lds<D>& sm, const f32x16 (&sacc)[4], f32x16 (&oacc)[D / 32]) {
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, l32 = lane & 31;
  bf16x8 pb[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const f32x16& s = sacc[kk >> 1];
    const int r0 = (kk & 1) * 8;
    pb[kk] = as_bf16x8(u32x4{pack_bf16x2(s[r0 + 0], s[r0 + 1]), pack_bf16x2(s[r0 + 2], s[r0 + 3]),
                             pack_bf16x2(s[r0 + 4], s[r0 + 5]), pack_bf16x2(s[r0 + 6], s[r0 + 7])});
  }
#pragma unroll
  for (int n = 0; n < D / 32; ++n) {
    __builtin_amdgcn_sched_barrier(0);
    oacc[n] = f32x16{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const uint16_t* vrow = &sm.vt[(n * 32 + l32) * Lds<D>::VP + half * 4];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + kk * 16);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + kk * 16 + 8);
      oacc[n] = mfma32(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pb[kk], oacc[n]);
    }
  }
}

// Row max (base-2 scaled scores in place), exponentials and row sum.
__device__ __forceinline__ void softmax_rows(f32x16 (&sacc)[4], float& m, float& l) {
  float mx = -__builtin_inff();
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[t][r]);
  mx = fmaxf(mx, swap_halves(mx));
  float sum = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(sacc[t][r] - mx);
      sacc[t][r] = e;
      sum += e;
    }
  sum += swap_halves(sum);
  m = mx;
  l = sum;
}

template <int D>
__device__ __forceinline__ void load_q(const uint16_t* __restrict__ qrow, bool valid, bf16x8 (&bq)[D / 16]) {
  const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    bq[ks] = as_bf16x8(valid ? load16(qrow + ks * 16 + half * 8) : u32x4{0u, 0u, 0u, 0u});
}

// ------------------------------------------------------------- kvouter pass

struct KvOuterArgs {
  Problem p;
  const uint16_t* q;
  const int32_t* entries;
  const int32_t* off;
  const int32_t* coff;
  const int32_t* chunk_list;
  uint16_t* part_o;
  float* part_st;
  int64_t n_lists;
  int hkv_shift;
  int chunk;
};

template <int D>
__global__ __launch_bounds__(256, 2) void kvouter_kernel(KvOuterArgs a) {
  __shared__ Lds<D> sm;
  const Problem& p = a.p;
  if ((int)blockIdx.x >= a.coff[a.n_lists]) return;
  const int list = a.chunk_list[blockIdx.x];
  const int e0 = a.off[list] + ((int)blockIdx.x - a.coff[list]) * a.chunk;
  const int e1 = min(e0 + a.chunk, a.off[list + 1]);
  const int phys = list >> a.hkv_shift;
  const int g = list & ((1 << a.hkv_shift) - 1);
  const int64_t key_stride = (int64_t)p.hkv * D;
  const int64_t base = ((int64_t)phys * kBlock * p.hkv + g) * D;
  stage_block<D>(sm, p.k + base, p.v + base, key_stride, kBlock);
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int G = p.group;
  const int rows = (e1 - e0) * G;
  for (int tile = wave; tile * 32 < rows; tile += 4) {
    const int rr = tile * 32 + l32;
    const bool valid = rr < rows;
    const int ei = valid ? rr / G : 0;
    const int hj = valid ? rr - ei * G : 0;
    const int code = valid ? a.entries[e0 + ei] : 0;
    const int64_t R = code >> 4;
    const int slot = code & 15;
    const int64_t r = R >> a.hkv_shift;
    bf16x8 bq[D / 16];
    load_q<D>(a.q + (r * p.hq + g * G + hj) * D, valid, bq);

    f32x16 sacc[4];
    block_scores<D>(sm, bq, sacc);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[t][i] *= p.scale_log2e;
    float m, l;
    softmax_rows(sacc, m, l);
    f32x16 oacc[D / 32];
    block_pv<D>(sm, sacc, oacc);

    // Normalised output, scaled by 2^-e into [-1, 1] for fp16 storage.
    const float inv_l = 1.0f / l;
    float amax = 0.f;
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        oacc[n][i] *= inv_l;
        amax = fmaxf(amax, fabsf(oacc[n][i]));
      }
    amax = fmaxf(amax, swap_halves(amax));
    const int ex = amax > 0.f ? (int)((__float_as_uint(amax) >> 23) & 0xff) - 126 : 0;
    const float f = ldexpf(1.0f, -ex);
    if (valid) {
      const int64_t pidx = (R * kSlots + slot) * G + hj;
      uint16_t* dst = a.part_o + pidx * D + half * 4;
#pragma unroll
      for (int n = 0; n < D / 32; ++n)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x16& o = oacc[n];
          *reinterpret_cast<u32x2*>(dst + n * 32 + q4 * 8) =
              u32x2{pack_f16x2(o[4 * q4] * f, o[4 * q4 + 1] * f), pack_f16x2(o[4 * q4 + 2] * f, o[4 * q4 + 3] * f)};
        }
      if (half == 0)
        *reinterpret_cast<f32x4*>(a.part_st + pidx * 4) = f32x4{m, l, (float)ex, 0.f};
    }
  }
}

// ----------------------------------------------- local block + merge pass

struct MergeArgs {
  Problem p;
  const uint16_t* q;
  const int32_t* sel;
  const uint16_t* part_o;
  const float* part_st;
  uint16_t* out;
  int hkv_shift;
};

constexpr int kMergeTq = 64;  // queries per merge workgroup (inside one block)

template <int D>
__global__ __launch_bounds__(256, 2) void merge_local_kernel(MergeArgs a) {
  __shared__ Lds<D> sm;
  const Problem& p = a.p;
  const int s = blockIdx.z, g = blockIdx.y;
  const int row0 = p.cu_q[s];
  const int nq = p.cu_q[s + 1] - row0;
  if (nq <= 0) return;
  const int seq_len = p.seq_lens[s];
  const int first_pos = seq_len - nq;
  const int tile0 = (first_pos / kMergeTq) * kMergeTq;
  const int n_tiles = (seq_len - 1 - tile0) / kMergeTq + 1;
  if ((int)blockIdx.x >= n_tiles) return;
  const int p0 = tile0 + blockIdx.x * kMergeTq;
  const int c = p0 >> 7;
  const int phys = p.block_table[(int64_t)s * p.max_blocks_per_seq + c];
  const bool phys_ok = phys >= 0 && phys < p.num_blocks;
  const int64_t key_stride = (int64_t)p.hkv * D;
  const int64_t base = ((int64_t)(phys_ok ? phys : 0) * kBlock * p.hkv + g) * D;
  stage_block<D>(sm, p.k + base, p.v + base, key_stride, phys_ok ? seq_len - c * kBlock : 0);
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int G = p.group;
  const int rows = kMergeTq * G;
  for (int tile = wave; tile * 32 < rows; tile += 4) {
    const int rr = tile * 32 + l32;
    const int qi = rr / G;
    const int hj = rr - qi * G;
    const int pos = p0 + qi;
    const bool valid = pos >= first_pos && pos < seq_len;
    const int64_t r = row0 + (int64_t)(pos - first_pos);
    const int h = g * G + hj;
    bf16x8 bq[D / 16];
    load_q<D>(a.q + (r * p.hq + h) * D, valid, bq);

    f32x16 sacc[4];
    block_scores<D>(sm, bq, sacc);
    const int lim = valid ? pos - c * kBlock : kBlock - 1;  // keys of the local block after the query are masked
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = t * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        sacc[t][i] = key <= lim ? sacc[t][i] * p.scale_log2e : -__builtin_inff();
      }
    float m_loc, l_loc;
    softmax_rows(sacc, m_loc, l_loc);
    f32x16 oacc[D / 32];
    block_pv<D>(sm, sacc, oacc);

    // Fold in the other selected blocks' partials (log-sum-exp merge): the
    // slots the kvouter pass wrote are exactly the non-local ids b < c of
    // slots 0..14 whose block is in the cache.
    const int64_t R = (r << a.hkv_shift) + g;
    uint32_t parts = 0;
    if (valid) {
      const int32_t* srow = a.sel + R * kTopK;
      const int32_t* table = p.block_table + (int64_t)s * p.max_blocks_per_seq;
      for (int j = 0; j < kSlots; ++j) {
        const int b = srow[j];
        if (b >= 0 && b < c) {
          const int pb = table[b];
          if (pb >= 0 && pb < p.num_blocks) parts |= 1u << j;
        }
      }
    }
    const float* st = a.part_st + (R * kSlots * G + hj) * 4;
    float M = m_loc;
    for (int j = 0; j < kSlots; ++j)
      if (parts >> j & 1u) M = fmaxf(M, st[(int64_t)j * G * 4]);
    const float w_loc = fast_exp2(m_loc - M);
    float L = l_loc * w_loc;
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[n][i] *= w_loc;
    for (int j = 0; j < kSlots; ++j) {
      if (!(parts >> j & 1u)) continue;
      const f32x4 sj = *reinterpret_cast<const f32x4*>(st + (int64_t)j * G * 4);
      const float w = sj[1] * fast_exp2(sj[0] - M);
      L += w;
      const float wy = ldexpf(w, (int)sj[2]);
      const uint16_t* y = a.part_o + ((R * kSlots + j) * G + hj) * D + half * 4;
#pragma unroll
      for (int n = 0; n < D / 32; ++n)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const u32x2 yv = *reinterpret_cast<const u32x2*>(y + n * 32 + q4 * 8);
          oacc[n][4 * q4 + 0] += wy * f16_lo(yv[0]);
          oacc[n][4 * q4 + 1] += wy * f16_hi(yv[0]);
          oacc[n][4 * q4 + 2] += wy * f16_lo(yv[1]);
          oacc[n][4 * q4 + 3] += wy * f16_hi(yv[1]);
        }
    }
    if (valid) {
      const float inv = 1.0f / L;
      uint16_t* dst = a.out + (r * p.hq + h) * D + half * 4;
#pragma unroll
      for (int n = 0; n < D / 32; ++n)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x16& o = oacc[n];
          *reinterpret_cast<u32x2*>(dst + n * 32 + q4 * 8) =
              u32x2{pack_bf16x2(o[4 * q4] * inv, o[4 * q4 + 1] * inv), pack_bf16x2(o[4 * q4 + 2] * inv, o[4 * q4 + 3] * inv)};
        }
    }
  }
}

// ------------------------------------------------------------------ launch

hipError_t launch_attn_prefill(const Problem& p, const uint16_t* q, const int32_t* sel, uint16_t* out, void* ws,
                               const int32_t* seq_lens_host, const int32_t* cu_q_host, hipStream_t stream) {
  if (p.total_q == 0) return hipSuccess;
  const PrefillWs w = prefill_layout(p);
  char* base = static_cast<char*>(ws);
  int hkv_shift = 0;
  while ((1 << hkv_shift) < p.hkv) ++hkv_shift;
  CsrArgs c{p, sel,
            reinterpret_cast<int32_t*>(base + w.cnt), reinterpret_cast<int32_t*>(base + w.off),
            reinterpret_cast<int32_t*>(base + w.coff), reinterpret_cast<int32_t*>(base + w.cursor),
            reinterpret_cast<int32_t*>(base + w.chunk_list), reinterpret_cast<int32_t*>(base + w.entries),
            w.n_lists, hkv_shift, w.chunk};
  const int64_t n_ent = ((int64_t)p.total_q << hkv_shift) * kTopK;
  const unsigned ent_blocks = (unsigned)((n_ent + 255) / 256);
  const unsigned list_blocks = (unsigned)((w.n_lists + 255) / 256);
  hipLaunchKernelGGL(csr_zero_kernel, dim3(std::min<unsigned>(list_blocks, 4096u)), dim3(256), 0, stream, c.cnt,
                     w.n_lists);
  hipLaunchKernelGGL(csr_count_kernel, dim3(ent_blocks), dim3(256), 0, stream, c);
  hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(1024), 0, stream, c);
  hipLaunchKernelGGL(csr_fill_kernel, dim3(ent_blocks), dim3(256), 0, stream, c);
  hipLaunchKernelGGL(csr_chunk_map_kernel, dim3(list_blocks), dim3(256), 0, stream, c);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  KvOuterArgs k{p, q, c.entries, c.off, c.coff, c.chunk_list,
                reinterpret_cast<uint16_t*>(base + w.part_o), reinterpret_cast<float*>(base + w.part_st),
                w.n_lists, hkv_shift, w.chunk};
  MergeArgs m{p, q, sel, k.part_o, k.part_st, out, hkv_shift};
  int max_tiles = 0;
  for (int s = 0; s < p.num_seqs; ++s) {
    const int nq = cu_q_host[s + 1] - cu_q_host[s];
    if (nq <= 0) continue;
    const int L = seq_lens_host[s];
    const int t0 = ((L - nq) / kMergeTq) * kMergeTq;
    max_tiles = std::max(max_tiles, (L - 1 - t0) / kMergeTq + 1);
  }
  const dim3 kv_grid((unsigned)w.max_chunks);
  const dim3 mg_grid((unsigned)max_tiles, (unsigned)p.hkv, (unsigned)p.num_seqs);
  if (p.head_dim == 128) {
    hipLaunchKernelGGL(kvouter_kernel<128>, kv_grid, dim3(256), 0, stream, k);
    hipLaunchKernelGGL(merge_local_kernel<128>, mg_grid, dim3(256), 0, stream, m);
  } else {
    hipLaunchKernelGGL(kvouter_kernel<64>, kv_grid, dim3(256), 0, stream, k);
    hipLaunchKernelGGL(merge_local_kernel<64>, mg_grid, dim3(256), 0, stream, m);
  }
  return hipGetLastError();
}

}  // namespace msa
