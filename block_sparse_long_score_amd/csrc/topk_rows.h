// topk_rows.h — the exp-free selection of one row's blocks, shared by the
// top-k kernels (block_topk.hip) and the fused decode step (attn_main.hip).
// Private to csrc/: not part of the C ABI.
//
// Source: "MiniMax 模型迭代与竞品分析：从 Text-01、M1、M2 到 M3", §2, MSA
// inference step 3 (16 blocks per query and group, the local block one of
// them); "MiniMax：Text-01 / M1 → M2.7 → M3", §5 (an exp-free Top-k).  Equal
// scores go to the lower block index; the algorithm is described at the top
// of block_topk.hip.
#pragma once

#include "msa_device.h"

namespace msa {

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// k-th largest of the 64 lane values (k <= 64): the largest T with
// |{lanes : x >= T}| >= k, built from the top bit down.  With LOW > 0 the
// LOW lowest bits are not searched: the result is the k-th largest with those
// bits cleared, a lower bound of it (the largest such T is at most the k-th
// largest, and every value above the k-th largest has a count below k).
template <int LOW = 0>
__device__ __forceinline__ uint32_t kth_largest_lane(uint32_t x, int k) {
  uint32_t t = 0;
#pragma unroll
  for (int bit = 31; bit >= LOW; --bit) {
    const uint32_t cand = t | (1u << bit);
    if (__popcll(__ballot(x >= cand)) >= k) t = cand;
  }
  return t;
}

constexpr int kKeep = kTopK - 1;  // non-local blocks kept per row
constexpr int kCached = 16;       // candidates per lane held in registers (rows with c <= 1024)

// Keys of candidates j*64 + lane for j in [j0, j0 + NC): one batch of
// independent loads (0 beyond the last candidate).  Each row is read once
// (or once per pass when streamed), so the loads are non-temporal.
template <int NC>
__device__ __forceinline__ void load_batch(const float* __restrict__ row, int c, int j0, uint32_t (&keys)[NC]) {
  const int lane = threadIdx.x & 63;
  float v[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int b = (j0 + j) * 64 + lane;
    v[j] = b < c ? __builtin_nontemporal_load(&row[b]) : 0.f;
  }
#pragma unroll
  for (int j = 0; j < NC; ++j) keys[j] = (j0 + j) * 64 + lane < c ? order_key(v[j]) : 0u;
}

// Selection for one row.  Rows with c <= 64 * NC candidates keep their keys
// in registers (one batch of loads); longer rows are streamed in batches of
// 64 * NC (NC per lane).  out_key (optional): each kept block's order key,
// beside its index in out.
template <bool CACHED, bool WRITE_LOCAL = true, int NC = kCached>
__device__ __forceinline__ void select_row(const float* __restrict__ row, int c, int32_t* __restrict__ out,
                                           uint32_t* surv_key, int32_t* surv_idx, uint32_t* out_key = nullptr) {
  const int lane = threadIdx.x & 63;
  const int nj = (c + 63) / 64;
  uint32_t keys[NC];
  if constexpr (CACHED) load_batch<NC>(row, c, 0, keys);

  // 1. lane maxima and theta.
  uint32_t lmax = 0;
  for (int j0 = 0; j0 < nj; j0 += NC) {
    if constexpr (!CACHED) load_batch<NC>(row, c, j0, keys);
#pragma unroll
    for (int j = 0; j < NC; ++j) lmax = max(lmax, keys[j]);
  }
  // A lower bound is all the compaction needs: the 16 high bits suffice.
  // Key 0 marks a lane past the row, so the bound is at least 1.
  const uint32_t theta = max(kth_largest_lane<16>(lmax, kKeep), 1u);

  // 2. compact survivors (key >= theta) in ascending block order.
  int count = 0;
  for (int j0 = 0; j0 < nj; j0 += NC) {
    if constexpr (!CACHED) load_batch<NC>(row, c, j0, keys);
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const bool ok = keys[j] >= theta;
      const uint64_t m = __ballot(ok);
      if (m != 0) {  // most groups hold no survivor: a ballot is all they cost
        const int pos = count + lanes_below(m);
        if (ok && pos < 64) {
          surv_key[pos] = keys[j];
          surv_idx[pos] = (j0 + j) * 64 + lane;
        }
        count += __popcll(m);
      }
    }
  }
  wave_lds_sync();

  if (count <= 64) {
    // 3. exact threshold among the survivors.
    const bool have = lane < count;
    const uint32_t k = have ? surv_key[lane] : 0u;
    const int idx = have ? surv_idx[lane] : 0;
    const uint32_t T = kth_largest_lane(k, kKeep);
    const int need = kKeep - __popcll(__ballot(have && k > T));
    const uint64_t eq = __ballot(have && k == T);
    const bool take = have && (k > T || (k == T && lanes_below(eq) < need));
    const uint64_t tm = __ballot(take);
    // 4. ascending output, local block last.
    if (take) {
      out[lanes_below(tm)] = idx;
      if (out_key) out_key[lanes_below(tm)] = k;
    }
  } else {
    // Massive ties: exact k-th largest over all candidates, bit by bit.
    auto key_at = [&](int j) -> uint32_t {
      const int b = j * 64 + lane;
      return b < c ? order_key(row[b]) : 0u;
    };
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      int n = 0;
      for (int j = 0; j < nj; ++j) n += __popcll(__ballot(key_at(j) >= cand));
      if (n >= kKeep) T = cand;
    }
    int gt = 0;
    for (int j = 0; j < nj; ++j) gt += __popcll(__ballot(key_at(j) > T));
    const int need = kKeep - gt;
    int taken = 0, ties = 0;
    for (int j = 0; j < nj && taken < kKeep; ++j) {
      const uint32_t k = key_at(j);
      const uint64_t eq = __ballot(k == T);
      const bool take = k > T || (k == T && ties + lanes_below(eq) < need);
      const uint64_t tm = __ballot(take);
      if (take) {
        out[taken + lanes_below(tm)] = j * 64 + lane;
        if (out_key) out_key[taken + lanes_below(tm)] = k;
      }
      taken += __popcll(tm);
      ties += __popcll(eq);
    }
  }
  if (WRITE_LOCAL && lane == 0) out[kKeep] = c;
}

// The top_k - 1 non-local blocks of one row with c > 15 candidates, chosen
// by the NW waves of a workgroup (every thread of the workgroup must call
// it): wave w finds the exact top 15 of its contiguous share of the
// candidates (ties to the lower index); the overall top 15 lies in the union
// of these, which wave 0 then searches in ascending block order with the same
// exact threshold and tie rule, writing out[0..15) ascending.  out may be
// global or LDS memory.  Each wave's candidates keep their keys beside their
// indices (cand, cand_key), so the union is searched without reading the row
// again.  The selection is unique, so it depends on neither NW nor NC (the
// candidates per lane each wave holds in registers).
template <int NW, int NC = kCached>
__device__ __forceinline__ void split_select_row(const float* __restrict__ row, int c, int32_t* out,
                                                 uint32_t (*surv_key)[64], int32_t (*surv_idx)[64],
                                                 int32_t (*cand)[kKeep], uint32_t (*cand_key)[kKeep]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Shares are multiples of 64 candidates; a share of n <= 15 keeps all n.
  const int share = ((c + NW * 64 - 1) / (NW * 64)) * 64;
  const int lo = min(c, wave * share), n = min(share, c - lo);
  if (n > 0) {
    if (n <= NC * 64)
      select_row<true, false, NC>(row + lo, n, cand[wave], surv_key[wave], surv_idx[wave], cand_key[wave]);
    else
      select_row<false, false, NC>(row + lo, n, cand[wave], surv_key[wave], surv_idx[wave], cand_key[wave]);
  }
  __syncthreads();
  if (wave != 0) return;
  // Candidates of all shares in ascending block order: up to NW * 15.
  constexpr int kRounds = (NW * kKeep + 63) / 64;
  uint32_t key[kRounds];
  int32_t idx[kRounds];
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const int e = j * 64 + lane;  // position in the concatenated list
    const int w = e / kKeep, k = e - w * kKeep;
    const int lo_w = min(c, w * share), n_w = min(share, c - lo_w);
    const bool have = w < NW && k < min(n_w, kKeep);
    idx[j] = have ? lo_w + cand[w][k] : -1;
    key[j] = have ? cand_key[w][k] : 0u;
  }
  // Exact 15th-largest key over the candidates, bit by bit.
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cnd = T | (1u << bit);
    int nge = 0;
#pragma unroll
    for (int j = 0; j < kRounds; ++j) nge += __popcll(__ballot(key[j] >= cnd));
    if (nge >= kKeep) T = cnd;
  }
  int gt = 0;
#pragma unroll
  for (int j = 0; j < kRounds; ++j) gt += __popcll(__ballot(key[j] > T));
  const int need = kKeep - gt;
  int taken = 0, ties = 0;
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const uint64_t eq = __ballot(key[j] == T && idx[j] >= 0);
    const bool take = idx[j] >= 0 && (key[j] > T || (key[j] == T && ties + lanes_below(eq) < need));
    const uint64_t tm = __ballot(take);
    if (take) out[taken + lanes_below(tm)] = idx[j];
    taken += __popcll(tm);
    ties += __popcll(eq);
  }
}

}  // namespace msa
