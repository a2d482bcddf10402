// msa_device.h — device-side helpers shared by the gfx950 kernels of libmsa.
// Private to csrc/: not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kBlock = 128;  // tokens per KV block
constexpr int kTopK = 16;    // blocks kept per query and group
constexpr int kWave = 64;    // CDNA wavefront width
// Cache-policy bits of a non-temporal load (gfx950 "nt").  Decode streams
// read-once data (the context's K_idx, the selected blocks' K/V, the partial
// rows) with it: 16 KB blocks in random order stream at ~6.5 TB/s this way
// against ~5.7 TB/s with plain loads.  Prefill keeps plain loads, because its
// K/V blocks and queries are read again soon enough for the Infinity Cache to
// serve some of them, but stores its partial rows (whole 128-byte lines,
// written once, read once) with the same bit.
constexpr int kLoadNT = 2;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> two bfloat16 packed in a uint32, round to nearest even
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Two floats -> two IEEE binary16 packed in a uint32, round to nearest even
// (one v_cvt_pk_f16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}

__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// Monotone map float -> uint32: a < b (as numbers) <=> key(a) < key(b).
// -0 is mapped like +0 so equal scores get equal keys.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 32x32x16 bf16 MFMA: D[32x32] += A[32x16] * B[16x32].
// Lane layout (wave64): A lane l holds A[l%32][8*(l/32) .. +7];
// B lane l holds B[8*(l/32) .. +7][l%32];
// D lane l, register r holds D[8*(r/4) + 4*(l/32) + (r%4)][l%32].
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Exchange a value with lane l^32 (the other half of the wave).
__device__ __forceinline__ float swap_halves(float v) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(((threadIdx.x & 63) ^ 32) << 2, __float_as_int(v)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// A 16-byte global-memory load from an address held as an integer.  A pointer
// rebuilt from an integer has no known address space, and the compiler would
// emit a flat load, which also counts against the LDS wait counter, so every
// later wait for an LDS read would wait for this load as well.
__device__ __forceinline__ u32x4 load16_global(uint64_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(addr);
}
__device__ __forceinline__ void store16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// Sequence of a query row: largest s with cu_q[s] <= row (cu_q ascending).
__device__ __forceinline__ int seq_of_row(const int32_t* __restrict__ cu_q, int num_seqs, int row) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace msa
