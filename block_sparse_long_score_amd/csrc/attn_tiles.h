// attn_tiles.h — MFMA tile pieces shared by the Main Branch kernels
// (attn_main.hip) and the dense causal attention kernel (dense_attn.hip).
// Private to csrc/: not part of the C ABI.
//
// MFMA mapping (32x32x16 bf16, wave64), per tile of 32 query rows and one
// 128-key block staged in LDS:
//   S^T[128 keys x 32 rows] = K[keys x D] * Q^T[D x rows]
//   O^T[D x 32 rows]        = V^T[D x keys] * P^T[keys x rows]
// With keys on the M axis each lane owns one row, so row max/sum are in-lane
// plus one exchange between wave halves, and the S^T accumulators rounded to
// bf16 are directly the B operand of the P.V product.  K and V are staged
// row-major, copied from the cache by the asynchronous global->LDS loads;
// the V^T operand comes from the LDS transpose load.
#pragma once

#include "msa_device.h"

namespace msa {

// One staged block: K and V of 128 keys, row-major [key][D], in 16-byte
// chunks placed at a per-row XOR of their index so that the operand reads
// touch every bank once per pass:
//   K (read as 16-byte rows of 16 keys x one chunk): slot = c ^ ((r/RPB) & (CPR-1));
//   V (read transposed, 4 keys x 4 chunks per 32 lanes): slot = c ^ (((r/RPB) & (CPR/4-1)) << 2),
// with CPR chunks per row and RPB rows per 256 bytes of banks.  For the rows
// a lane reads, both XOR terms depend on the lane only, so every operand
// address is a per-lane base plus a compile-time offset.
template <int D>
__device__ __forceinline__ int kv_kslot(int r, int c) {
  constexpr int CPR = D / 8, RPB = 128 / D;
  return c ^ ((r / RPB) & (CPR - 1));
}

template <int D>
__device__ __forceinline__ int kv_vslot(int r, int c) {
  constexpr int CPR = D / 8, RPB = 128 / D;
  return c ^ (((r / RPB) & (CPR / 4 - 1)) << 2);
}

// Per-lane byte offsets of the block copy by a workgroup of WAVES waves:
// round i moves slots (WAVES*i + wave) * 64 + lane of K and of V (row
// r = slot / CPR), reading the global chunk that belongs in that slot.
template <int D, int WAVES>
struct DmaLane {
  static constexpr int CPR = D / 8;
  static constexpr int ROUNDS = kBlock * CPR / (64 * WAVES);
  uint32_t koff[ROUNDS], voff[ROUNDS];  // bytes from the block's first key row
  int row[ROUNDS];
};

template <int D, int WAVES>
__device__ __forceinline__ DmaLane<D, WAVES> dma_lane(int wave, int lane, int64_t key_stride) {
  DmaLane<D, WAVES> d;
#pragma unroll
  for (int i = 0; i < DmaLane<D, WAVES>::ROUNDS; ++i) {
    const int slot_idx = (i * WAVES + wave) * 64 + lane;
    const int r = slot_idx / DmaLane<D, WAVES>::CPR, sl = slot_idx % DmaLane<D, WAVES>::CPR;
    d.row[i] = r;
    d.koff[i] = (uint32_t)((r * key_stride + kv_kslot<D>(r, sl) * 8) * 2);
    d.voff[i] = (uint32_t)((r * key_stride + kv_vslot<D>(r, sl) * 8) * 2);
  }
  return d;
}

// Asynchronous copy of the K rows (V = false) or V rows (V = true) of one
// block of group g into a 128 x D LDS matrix with the global->LDS loads
// (each wave instruction fills 64 consecutive 16-byte slots).  In a block
// cut short by the end of the sequence, keys at or after `valid` read the
// last valid key instead: finite data, and always masked since they lie
// after every query position that reads them.
template <int D, int WAVES, bool V>
__device__ __forceinline__ void block_dma(uint16_t* dst, const DmaLane<D, WAVES>& dl, int wave, const uint16_t* src,
                                          int64_t key_stride, int valid) {
  const char* sb = reinterpret_cast<const char*>(src);
  const bool full = valid == kBlock;
#pragma unroll
  for (int i = 0; i < DmaLane<D, WAVES>::ROUNDS; ++i) {
    const int run = i * WAVES + wave;
    uint32_t off = V ? dl.voff[i] : dl.koff[i];
    if (!full && dl.row[i] >= valid) off -= (uint32_t)((dl.row[i] - (valid - 1)) * key_stride * 2);
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(sb + off),
                                     reinterpret_cast<__attribute__((address_space(3))) void*>(
                                         reinterpret_cast<uintptr_t>(dst + run * 512)),
                                     16, 0, 0);
  }
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Transposed LDS read (gfx950 ds_read_b64_tr_b16): within each group of 16
// lanes, lane 4a+b receives element b of the 4-element row addressed by
// lane 4j+a, for j = 0..3.
typedef __attribute__((address_space(3))) const char lds_byte;

// An LDS buffer's address as a run-time value: the operand reads then add
// one per-lane base to it and fold their constant offsets (a buffer placed
// at 64 KB or above would otherwise need an extra add per read, its address
// exceeding the 16-bit offset field).
__device__ __forceinline__ lds_byte* opaque_lds(const uint16_t* p) {
  uint32_t a = (uint32_t)reinterpret_cast<uintptr_t>((lds_byte*)p);
  asm volatile("" : "+s"(a));
  return (lds_byte*)(uintptr_t)a;
}

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
  for (int ks = 0; ks < D / 16; ++ks) o.k[ks] = (uint32_t)((l32 * D + kv_kslot<D>(l32, 2 * ks + half) * 8) * 2);
  const int gi = lane >> 4, s16 = lane & 15;
  const int jr = s16 >> 2, a4 = s16 & 3;
  const int r = 4 * (gi >> 1) + jr;
#pragma unroll
  for (int n = 0; n < D / 32; ++n) {
    const int c = 4 * n + 2 * (gi & 1) + (a4 >> 1);
    o.v[n] = (uint32_t)((r * D + kv_vslot<D>(r, c) * 8 + (a4 & 1) * 4) * 2);
  }
  return o;
}

// S^T = K Q^T of one staged block for this wave's 32 rows (4 key tiles).
// The K operands of k-step ks+1 are read while the products of step ks run.
template <int D>
__device__ __forceinline__ void tile_scores(lds_byte* kb, const OpLane<D>& ol, const bf16x8 (&bq)[D / 16],
                                            f32x16 (&sacc)[4]) {
  __builtin_amdgcn_sched_barrier(0);  // phases are scheduled apart: bounds live operand registers
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4)
    sacc[t4] = f32x16{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto rd = [&](int ks, int t4) {
    return *reinterpret_cast<__attribute__((address_space(3))) const u32x4*>(kb + ol.k[ks] + t4 * 32 * D * 2);
  };
  u32x4 cur[4], nxt[4];
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4) cur[t4] = rd(0, t4);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    if (ks + 1 < D / 16)
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) nxt[t4] = rd(ks + 1, t4);
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) sacc[t4] = mfma32(as_bf16x8(cur[t4]), bq[ks], sacc[t4]);
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) cur[t4] = nxt[t4];
  }
}

// O^T = V^T P^T (ACC: O^T += V^T P^T) for one staged block.  The V^T
// operands of k-step kk+1 are read while the products of step kk run.
template <int D, bool ACC>
__device__ __forceinline__ void tile_pv(lds_byte* vb, const OpLane<D>& ol, const bf16x8 (&pb)[8],
                                        f32x16 (&oacc)[D / 32]) {
  __builtin_amdgcn_sched_barrier(0);
  if (!ACC)
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
      oacc[n] = f32x16{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  constexpr int NT = D / 32;
  auto rd = [&](int kk, int n) {
    const i16x4 lo = lds_read_tr16(vb + ol.v[n] + (16 * kk) * D * 2);
    const i16x4 hi = lds_read_tr16(vb + ol.v[n] + (16 * kk + 8) * D * 2);
    const u32x2 lw = __builtin_bit_cast(u32x2, lo), hw = __builtin_bit_cast(u32x2, hi);
    return u32x4{lw[0], lw[1], hw[0], hw[1]};
  };
  u32x4 cur[NT], nxt[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) cur[n] = rd(0, n);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    if (kk + 1 < 8)
#pragma unroll
      for (int n = 0; n < NT; ++n) nxt[n] = rd(kk + 1, n);
#pragma unroll
    for (int n = 0; n < NT; ++n) oacc[n] = mfma32(as_bf16x8(cur[n]), pb[kk], oacc[n]);
#pragma unroll
    for (int n = 0; n < NT; ++n) cur[n] = nxt[n];
  }
}

// P (the exponentiated S^T accumulators) rounded to bf16 in the key order
// of the P^T operand: k-step kk holds accumulator registers 8(kk%2)..+7 of
// key tile kk/2.
__device__ __forceinline__ void p_operand(const f32x16 (&sacc)[4], bf16x8 (&pb)[8]) {
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const f32x16& s = sacc[kk >> 1];
    const int r0 = (kk & 1) * 8;
    pb[kk] = as_bf16x8(u32x4{pack_bf16x2(s[r0 + 0], s[r0 + 1]), pack_bf16x2(s[r0 + 2], s[r0 + 3]),
                             pack_bf16x2(s[r0 + 4], s[r0 + 5]), pack_bf16x2(s[r0 + 6], s[r0 + 7])});
  }
}

// Softmax statistics of 32 rows over the staged block, in base 2: with raw
// scores s and c = softmax_scale * log2(e) > 0, m = c * max(s) and
// p = 2^(c*s - m) (one FMA and one exp per score).  p replaces s in place;
// masked scores are -inf and give p = 0.
__device__ __forceinline__ void softmax_rows(f32x16 (&sacc)[4], float c, float& m, float& l) {
  float mx = -__builtin_inff();
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[t][r]);
  mx = fmaxf(mx, swap_halves(mx)) * c;
  float sum = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(fmaf(sacc[t][r], c, -mx));
      sacc[t][r] = e;
      sum += e;
    }
  sum += swap_halves(sum);
  m = mx;
  l = sum;
}

// Query rows of a 32-row tile as the B operand of tile_scores: lane (row
// rho, half h) needs dims 16*ks + 8h .. +7 of row rho for every k-step ks,
// 16 bytes at byte 32*ks + 16h of its own row, so the loads land in operand
// order (one address per lane, the k-steps as immediate offsets; the two
// lanes of a row read 32 consecutive bytes per load).  Loads are issued early
// (load_q_raw, into registers the next tile's math does not touch) and taken
// as the operand when it is needed (q_operand).
template <int D>
struct QRaw {
  u32x4 q[D / 16];
};

template <int D>
__device__ __forceinline__ void load_q_raw(const uint16_t* __restrict__ qrow, QRaw<D>& raw) {
  const int h = (threadIdx.x >> 5) & 1;
  const uint64_t base = reinterpret_cast<uint64_t>(qrow) + (uint64_t)(16 * h);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) raw.q[ks] = load16_global(base + (uint64_t)(32 * ks));
}

template <int D>
__device__ __forceinline__ void q_operand(const QRaw<D>& raw, bf16x8 (&bq)[D / 16]) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) bq[ks] = as_bf16x8(raw.q[ks]);
}

// ------------------------------------------------------ decode, one wave

// A raw buffer resource over `bytes` bytes from `base` (gfx9 descriptor
// word 3); loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One wave attends a decode query's G heads (G <= GM <= 16) to the keys of
// one block after another, keeping a running softmax state.  Scores use the
// 16x16x32 bf16 MFMA with 16 keys on M (K rows staged in the wave's LDS
// region) and the heads on N (padded to 16); P.V uses vector ALU math with each lane
// owning D/64 output dims.  16x16x32 lane layout: A lane l holds
// A[l%16][8*(l/16) .. +7], B lane l holds B[8*(l/16) .. +7][l%16], D lane l
// register i holds D[4*(l/16) + i][l%16].
// Steps of 16 keys, software-pipelined for G <= 8: the K and V rows of the
// next step are requested before the current step is multiplied, so every
// wave keeps loads in flight while it computes (two register sets of V, one
// LDS region of K).  A step's 16 K rows reach the wave's own LDS region by
// direct global-to-LDS loads of whole rows (each load instruction moves
// 64 / (D/8) rows of D*2 contiguous bytes; 16-byte chunks XOR-swizzled by
// row), and the A operand is read from there: loaded straight into operand
// order, each instruction would read only 64 bytes of each of 16 rows.
template <int D, int GM>
struct DecodeWave {
  static constexpr int VPL = D / 64;            // output dims per lane in P.V
  static constexpr int KS = D / 32;             // MFMA k-steps
  static constexpr int SUB = 16;                // keys per online-softmax step
  static constexpr int NSTEP = kBlock / SUB;
  static constexpr int CPR = D / 8;             // 16-byte chunks per K row
  static constexpr int RPI = 64 / CPR;          // K rows per load instruction
  static constexpr int STAGE = SUB * D;         // bf16 elements of a step's staged K rows
  static_assert(SUB == 16, "the partial waits below are written as vmcnt(16)");
  // Chunk c of staged row r sits at chunk position c ^ swz(r): a step's 16
  // rows then cover every bank once for any one logical chunk.
  static __device__ __forceinline__ int swz(int r) { return (r / (256 / (D * 2))) & (CPR - 1); }  // D <= 128
  // At G > 8 the 16 heads' accumulators leave no registers for a second step in flight.
  static constexpr bool kPipelined = GM <= 8;
  float m_run = -__builtin_inff(), l_run = 0.f;  // head l16's running max (base 2) and sum
  float acc[GM][VPL];

  __device__ DecodeWave() {
#pragma unroll
    for (int j = 0; j < GM; ++j)
#pragma unroll
      for (int v = 0; v < VPL; ++v) acc[j][v] = 0.f;
  }

  // The B operand: head l16 of the group (heads G.. are zero), dims of k-step ks.
  // Loads read from in-range addresses unconditionally and zero what is out
  // of range afterwards, so they issue as one batch without branches.
  __device__ __forceinline__ void load_q(const uint16_t* q_group, int G, bf16x8 (&bq)[KS]) const {
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15, q16 = lane >> 4;
    const bool head_ok = l16 < G;
    const uint16_t* qh = q_group + (int64_t)min(l16, G - 1) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 x = load16(qh + ks * 32 + q16 * 8);
      bq[ks] = as_bf16x8(head_ok ? x : u32x4{0u, 0u, 0u, 0u});
    }
  }

  // Requests (non-temporal loads), into the wave's LDS region `stage`, the K
  // rows of keys [c0, c0 + 16) and then the V rows (lane: dims lane*VPL ..);
  // keys at or past nvalid read key nvalid-1.  The K copies go first, so a
  // wait for all but the last SUB (= 16, one per V row) memory operations of
  // the wave covers them while the V rows may still be in flight.  kg: the block-head's first K
  // row; vr: a buffer resource over its V rows; ks_b: the key stride in
  // bytes.  A V row's offset is the same in every lane (a scalar offset);
  // each lane adds only its own dims.
  __device__ __forceinline__ void issue(const uint16_t* kg, __amdgpu_buffer_rsrc_t vr, int ks_b, int nvalid, int c0,
                                        uint32_t (&vreg)[SUB], uint16_t* stage) const {
    const int lane = threadIdx.x & 63;
    const char* kb = reinterpret_cast<const char*>(kg);
#pragma unroll
    for (int j = 0; j < SUB / RPI; ++j) {
      const int r = j * RPI + lane / CPR;  // staged row; lane's chunk position lane % CPR
      const int chunk = (lane % CPR) ^ swz(r);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(kb + (int64_t)min(c0 + r, nvalid - 1) * ks_b + chunk * 16),
                                       reinterpret_cast<__attribute__((address_space(3))) void*>(
                                           reinterpret_cast<uintptr_t>(stage + j * 512)),
                                       16, 0, kLoadNT);
    }
#pragma unroll
    for (int kk = 0; kk < SUB; ++kk) {
      const int soff = min(c0 + kk, nvalid - 1) * ks_b;
      if constexpr (VPL == 2)
        vreg[kk] = __builtin_amdgcn_raw_buffer_load_b32(vr, lane * 4, soff, kLoadNT);
      else
        vreg[kk] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(vr, lane * 2, soff, kLoadNT);
    }
  }

  // The A operand of a staged step: lane (key l16, q16) takes logical chunk
  // 4*ks + q16 of its key's row.
  __device__ __forceinline__ void read_k(const uint16_t* stage, bf16x8 (&ak)[KS]) const {
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15, q16 = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      ak[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(&stage[l16 * D + (((4 * ks + q16) ^ swz(l16)) * 8)]));
  }

  // One step: scores of keys [c0, c0 + 16), the running softmax, and P.V.
  __device__ __forceinline__ void step(int nvalid, int c0, const uint32_t (&vreg)[SUB], const bf16x8 (&ak)[KS],
                                       const bf16x8 (&bq)[KS], float c, float (&p_w)[GM][SUB],
                                       float (&alpha_w)[GM]) {
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15, q16 = lane >> 4;
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[ks], bq[ks], sacc, 0, 0, 0);
    // lane (head l16, q16) holds keys c0 + 4*q16 + i
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = c0 + 4 * q16 + i < nvalid ? sacc[i] : -__builtin_inff();
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * c);  // finite: key c0 is valid
    const float alpha = fast_exp2(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pe = fast_exp2(fmaf(sc[i], c, -m_new));
      psum += pe;
      if (l16 < GM) p_w[l16][4 * q16 + i] = pe;
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l_run = fmaf(l_run, alpha, psum);
    m_run = m_new;
    if (q16 == 0 && l16 < GM) alpha_w[l16] = alpha;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
    for (int j = 0; j < GM; ++j) {
      const float al = alpha_w[j];
#pragma unroll
      for (int vv = 0; vv < VPL; ++vv) acc[j][vv] *= al;
    }
#pragma unroll
    for (int k4 = 0; k4 < SUB / 4; ++k4) {
      float vf[4][VPL];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // keys past nvalid carry p = 0; their V (a valid row's) is zeroed too
        const uint32_t w = c0 + k4 * 4 + i < nvalid ? vreg[k4 * 4 + i] : 0u;
        vf[i][0] = bf16_to_f32(w & 0xffffu);
        if constexpr (VPL == 2) vf[i][1] = bf16_to_f32(w >> 16);
      }
#pragma unroll
      for (int j = 0; j < GM; ++j) {
        const f32x4 pj = *reinterpret_cast<const f32x4*>(&p_w[j][k4 * 4]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int vv = 0; vv < VPL; ++vv) acc[j][vv] = fmaf(pj[i], vf[i][vv], acc[j][vv]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }

  // Keys [0, nvalid) of the block whose head-g rows start at k + base / v + base
  // (1 <= nvalid <= 128).  p_w, alpha_w: this wave's LDS scratch for the P rows
  // and the rescale factors; stage: its LDS region of STAGE bf16 for the K
  // rows.  PIPE: request the next step before the current one is multiplied
  // (needs the second register set).  Every request has landed on return.
  template <bool PIPE = kPipelined>
  __device__ __forceinline__ void attend_block(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                               int64_t base, int64_t key_stride, int nvalid, const bf16x8 (&bq)[KS],
                                               float c, float (&p_w)[GM][SUB], float (&alpha_w)[GM], uint16_t* stage) {
    const int ks_b = (int)(key_stride * 2);
    const uint32_t bytes = (uint32_t)((kBlock - 1) * ks_b + D * 2);
    const __amdgpu_buffer_rsrc_t vb = buffer_rsrc(v + base, bytes);
    const uint16_t* kg = k + base;
    if constexpr (PIPE) {
      uint32_t vreg[2][SUB];
      issue(kg, vb, ks_b, nvalid, 0, vreg[0], stage);
#pragma unroll
      for (int st = 0; st < NSTEP; ++st) {
        const int c0 = st * SUB;
        if (c0 >= nvalid) break;
        bf16x8 ak[KS];
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");  // this step's K rows have landed (its 16 V rows may not)
        read_k(stage, ak);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before the region is refilled
        if (st + 1 < NSTEP) issue(kg, vb, ks_b, nvalid, c0 + SUB, vreg[(st + 1) & 1], stage);
        step(nvalid, c0, vreg[st & 1], ak, bq, c, p_w, alpha_w);
      }
    } else {
      for (int c0 = 0; c0 < nvalid; c0 += SUB) {
        uint32_t vreg[SUB];
        bf16x8 ak[KS];
        issue(kg, vb, ks_b, nvalid, c0, vreg, stage);
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");  // the K rows have landed (the 16 V rows may not)
        read_k(stage, ak);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before the region is refilled
        step(nvalid, c0, vreg, ak, bq, c, p_w, alpha_w);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
  }

  // This wave's unnormalised output rows and softmax state into LDS for the
  // combine (-inf and 0 for a wave that attended nothing).
  __device__ __forceinline__ void store(float (&o_w)[GM][D], float (&m_w)[GM], float (&l_w)[GM]) const {
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15, q16 = lane >> 4;
#pragma unroll
    for (int j = 0; j < GM; ++j)
#pragma unroll
      for (int v = 0; v < VPL; ++v) o_w[j][lane * VPL + v] = acc[j][v];
    if (q16 == 0 && l16 < GM) {
      m_w[l16] = m_run;
      l_w[l16] = l_run;
    }
  }
};

// Log-sum-exp combine of NW waves' states for head j, dims d and d+1: the
// unnormalised sums (o0, o1) and the mass L, both relative to 2^M.
template <int D, int GM, int NW>
__device__ __forceinline__ void combine_waves(const float (&o_s)[NW][GM][D], const float (&m_s)[NW][GM],
                                              const float (&l_s)[NW][GM], int j, int d, float& o0, float& o1,
                                              float& L, float& M) {
  M = -__builtin_inff();
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, m_s[ww][j]);
  L = 0.f;
  o0 = 0.f;
  o1 = 0.f;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) {
    const float f = l_s[ww][j] > 0.f ? fast_exp2(m_s[ww][j] - M) : 0.f;
    L = fmaf(l_s[ww][j], f, L);
    o0 = fmaf(o_s[ww][j][d], f, o0);
    o1 = fmaf(o_s[ww][j][d + 1], f, o1);
  }
}

}  // namespace msa
