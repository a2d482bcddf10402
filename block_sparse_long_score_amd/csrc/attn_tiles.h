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
// bf16 are directly the B operand of the P.V product; V is stored transposed
// in LDS so its A operand is two 8-byte reads.
#pragma once

#include "msa_device.h"

namespace msa {

template <int D>
struct Lds {
  static constexpr int KP = D + 8;    // K row pitch (bf16): rows stay 16-byte aligned
  static constexpr int VP = 128 + 4;  // V^T row pitch (bf16): 66 words, so the 32 rows one PV operand read touches fill all 64 banks once
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

// O^T = V^T P^T for 32 rows (ACC: O^T += V^T P^T); P given by the
// (exponentiated) S^T accumulators.
template <int D, bool ACC = false>
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
    if (!ACC) oacc[n] = f32x16{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const uint16_t* vrow = &sm.vt[(n * 32 + l32) * Lds<D>::VP + half * 4];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + kk * 16);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + kk * 16 + 8);
      oacc[n] = mfma32(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pb[kk], oacc[n]);
    }
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

// Query rows of a 32-row tile as the B operand of block_scores: lane (row
// rho, half h) needs dims 16*ks + 8h .. +7 of row rho for every k-step ks.
// They are loaded as 64-byte row segments: in load pair j, lane (h, a, b)
// (a = bit 4 of the lane, b its low 4 bits) reads 16 bytes of tile row b
// (first load) and of tile row 16 + b (second load), so four lanes cover 32
// consecutive dims of one row per load.  q_operand() then swaps with the
// lane 16 away to give every lane its own row.  Loads are issued early
// (load_q_raw) and the swaps done when the operand is needed.
template <int D>
struct QRaw {
  u32x4 a[D / 32], b[D / 32];
};

__device__ __forceinline__ uint32_t partner16(uint32_t x) {
  const auto t = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return (threadIdx.x & 16) ? t[0] : t[1];
}

template <int D>
__device__ __forceinline__ void load_q_raw(const uint16_t* __restrict__ qrow, QRaw<D>& raw) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, a16 = (lane >> 4) & 1;
  const uint64_t own = reinterpret_cast<uint64_t>(qrow);
  const uint64_t other = ((uint64_t)partner16((uint32_t)(own >> 32)) << 32) | partner16((uint32_t)own);
  const uint16_t* rowA = reinterpret_cast<const uint16_t*>(a16 ? other : own);  // tile row b
  const uint16_t* rowB = reinterpret_cast<const uint16_t*>(a16 ? own : other);  // tile row 16 + b
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    raw.a[j] = load16(rowA + (4 * j + 2 * a16 + h) * 8);
    raw.b[j] = load16(rowB + (4 * j + 2 * (1 - a16) + h) * 8);
  }
}

template <int D>
__device__ __forceinline__ void q_operand(const QRaw<D>& raw, bf16x8 (&bq)[D / 16]) {
  const bool a16 = (threadIdx.x & 16) != 0;
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    u32x4 x, y;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto t = __builtin_amdgcn_permlane16_swap(raw.a[j][i], raw.b[j][i], false, false);
      x[i] = a16 ? t[1] : t[0];  // dims 32j + 8h .. +7 of this lane's row
      y[i] = a16 ? t[0] : t[1];  // dims 32j + 16 + 8h .. +7
    }
    bq[2 * j] = as_bf16x8(x);
    bq[2 * j + 1] = as_bf16x8(y);
  }
}

}  // namespace msa
