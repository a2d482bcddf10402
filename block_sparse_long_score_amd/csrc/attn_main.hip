// attn_main.hip — Main Branch of MSA: exact softmax attention of every query
// row over the tokens of its selected blocks, for prefill and decode.
//
// Source: "MiniMax 模型迭代与竞品分析：从 Text-01、M1、M2 到 M3", §2: the
// softmax-attention equation (scores q.k/sqrt(d_k), softmax over the attended
// keys, probability-weighted sum of values) and MSA step 4 (standard softmax
// attention restricted to the chosen blocks, at most 16 x 128 = 2048 tokens).
// "MiniMax：Text-01 / M1 → M2.7 → M3", §5 names a KV-outer kernel design for
// the block-level irregular access; "前沿架构解码手记（三）" §2.1 motivates the
// block-major cache: a chosen block is one contiguous piece per head.
//
// Schedule (blocks outer).  The up-to-16 blocks a (query, group) row selects
// are scattered, so queries that share a block are scattered too: gathering
// the blocks per query would move 1 MB of K/V per (query, group) at head_dim
// 128.  Instead every (block, group) pair is loaded into LDS once per chunk of
// the queries that selected it:
//   prefill  1. invert the selections into one list of (row, slot) entries per
//               (sequence, group, logical block): an LDS histogram per chunk of
//               512 query rows, a column scan over the chunks, a scan over the
//               lists, and a scatter (no global atomics);
//            2. kvouter: one workgroup per chunk of a list stages the block's K
//               and V in LDS and runs every listed row's heads against it with
//               bf16 MFMA; rows whose local block this is mask the keys after
//               the query.  Output per (row, slot, head): block-local softmax
//               statistics and the normalised output in fp16 scaled by 2^-e;
//   decode   batches of >= 128 (sequence, group) pairs: decode_fused, one
//               16-wave workgroup per pair, one wave per selected block, waves
//               combined in LDS, output written directly; smaller batches:
//               decode_block, one workgroup per (slot, group, sequence), no
//               staging, then the merge below;
//   prefill  3. merge: per (row, head) a streaming log-sum-exp over the slots,
//   (and small decode) rounded to bf16.
// The softmax works in base 2 with the scale folded into log2(e).
//
// MFMA mapping (32x32x16 bf16, wave64), per tile of 32 (row, head) pairs:
//   S^T[128 keys x 32 rows] = K[keys x D] * Q^T[D x rows]   (K from LDS, Q from HBM)
//   O^T[D x 32 rows]        = V^T[D x keys] * P^T[keys x rows]
// With keys on the M axis each lane owns one row, so row max/sum are in-lane
// plus one exchange between wave halves, and the S^T accumulators rounded to
// bf16 are directly the B operand of the P.V product.  The block's K and V
// are staged row-major by asynchronous global->LDS copies; the V^T operand
// is read with the LDS transpose load (attn_tiles.h).
#include <mutex>

#include "attn_tiles.h"
#include "msa_kernels.h"
#include "topk_rows.h"

namespace msa {

constexpr int kCsrRows = 512;  // query rows per selection-inversion workgroup

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int hkv_shift_of(const Problem& p) {
  int s = 0;
  while ((1 << s) < p.hkv) ++s;
  return s;
}

// Entries (row, slot) per kvouter workgroup: ~3072 (row, head) pairs, so
// each staged block serves ~96 row tiles before it is dropped (a list of a
// 16384-row chunk at 128K context fits one workgroup).
constexpr int kKvMaxChunk = 3072;  // (entry, head) rows per kvouter workgroup, at most
static int kv_chunk(const Problem& p) { return std::max(16, kKvMaxChunk / p.group); }

// Decode batches with at least this many (sequence, group) pairs give each
// pair whole 16-wave workgroups (any G <= 16); smaller ones split each pair
// over 16 workgroups (one per selected block) and merge.
constexpr int64_t kFusedDecodeMinGroups = 128;
// Batches with fewer pairs than this (and at least kFusedDecodeMinGroups)
// give each pair two workgroups (decode_fused_half_kernel), so that every CU
// streams; larger ones one (decode_fused_kernel).  Both the decode call and
// the fused decode step follow this split.
constexpr int64_t kFusedHalfMaxGroups = 256;

// ---------------------------------------------------------------- workspace

// Two regions: the plan (prefill only: the selection inversion) and the
// partial outputs.  Offsets are relative to the start of their own region.
struct MainWs {
  size_t cnt_mat, list_cnt, off, coff, chunk_list, entries, entry_of, plan_total;
  size_t part_o, part_st, part_total;
  int64_t n_lists, max_entries, max_kv_chunks;
  int csr_chunks;  // row chunks per sequence (grid x of the inversion kernels)
  int chunk;       // entries per kvouter workgroup
};

static MainWs main_layout(const Problem& p, bool decode) {
  MainWs w{};
  const int64_t parts = (int64_t)p.total_q * p.hkv * kTopK * p.group;
  size_t o = 0;
  if (!decode) {
    w.chunk = kv_chunk(p);
    w.csr_chunks = std::max(1, (p.max_q_per_seq + kCsrRows - 1) / kCsrRows);
    w.n_lists = (int64_t)p.num_seqs * p.hkv * p.max_blocks_per_seq;
    w.max_entries = (int64_t)p.total_q * p.hkv * kTopK;
    w.max_kv_chunks = (w.max_entries + w.chunk - 1) / w.chunk + std::min<int64_t>(w.n_lists, w.max_entries);
    w.cnt_mat = o;    o = align256(o + sizeof(int32_t) * w.n_lists * w.csr_chunks);
    w.list_cnt = o;   o = align256(o + sizeof(int32_t) * w.n_lists);
    w.off = o;        o = align256(o + sizeof(int32_t) * (w.n_lists + 1));
    w.coff = o;       o = align256(o + sizeof(int32_t) * (w.n_lists + 1));
    w.chunk_list = o; o = align256(o + sizeof(int32_t) * (w.max_kv_chunks + 1));
    w.entries = o;    o = align256(o + sizeof(int32_t) * (w.max_entries + 1));
    w.entry_of = o;   o = align256(o + sizeof(int32_t) * w.max_entries);
  }
  w.plan_total = o;
  o = 0;
  w.part_o = o;  o = align256(o + sizeof(uint16_t) * parts * p.head_dim);
  w.part_st = o; o = align256(o + sizeof(float) * 2 * parts);
  w.part_total = o;
  return w;
}

size_t prefill_plan_bytes(const Problem& p) { return main_layout(p, false).plan_total; }
size_t prefill_run_bytes(const Problem& p) { return main_layout(p, false).part_total; }
size_t prefill_workspace_bytes(const Problem& p) {
  const MainWs w = main_layout(p, false);
  return w.plan_total + w.part_total;
}
size_t decode_workspace_bytes(const Problem& p) { return main_layout(p, true).part_total; }

// The two-workgroup decode (decode_fused_half_kernel) keeps, at the start of
// the partial region, each (pair, half)'s G x D output sums and G (max, mass)
// pairs, then one counter per pair; this always fits in the region, which
// holds 16 fp16 partial rows per (pair, head).
static size_t decode_half_state_bytes(const Problem& p) {
  return align256(sizeof(float) * (size_t)p.total_q * p.hkv * 2 * ((size_t)p.group * p.head_dim + 2 * p.group));
}
static bool decode_uses_half(const Problem& p) {
  const int64_t pairs = (int64_t)p.num_seqs * p.hkv;
  return pairs >= kFusedDecodeMinGroups && pairs < kFusedHalfMaxGroups;
}

// ------------------------------------------------- decode without allocation

// The split decode (fewer than kFusedDecodeMinGroups (sequence, group) pairs)
// keeps one partial row per (pair, slot, head) in scratch memory; batches of
// up to kFusedHalfMaxGroups pairs keep two halves' G x D sums per pair and a
// counter (at most 255 * 2 * (16 * 128 + 32) floats, about 4.2 MB); larger
// batches use decode_fused_kernel, which needs none.  So the scratch of the
// largest split decode, 127 pairs at G = 16 and D = 128, serves every decode
// batch: 127 * 16 * 16 partial rows of 128 fp16 values and 8 bytes of
// statistics each.
constexpr size_t kDecodeScratchBytes = ((size_t)127 * 16 * 16 * 128 * 2 + 255) / 256 * 256 +
                                       ((size_t)127 * 16 * 16 * 2 * 4 + 255) / 256 * 256;

// The scratch of msa_sparse_attn_decode_noalloc.  Each GPU holds its own copy
// from the library's first use on it until the process ends.  Host code never
// uses this name as an address (on the host it is only a stand-in for the
// symbol): kernels receive the device address that decode_scratch() looked up
// for the GPU they run on.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

size_t decode_scratch_capacity() { return kDecodeScratchBytes; }

size_t decode_scratch_need(const Problem& p) {
  if (decode_uses_half(p)) return decode_half_state_bytes(p) + sizeof(int32_t) * (size_t)p.total_q * p.hkv;
  return (int64_t)p.num_seqs * p.hkv >= kFusedDecodeMinGroups ? 0 : decode_workspace_bytes(p);
}

// Device address of `scratch` on `device`, looked up once per device (with
// that device current) and kept for the life of the process.
hipError_t decode_scratch(int device, void** addr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* table[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!table[device]) {
    int current = 0;
    hipError_t e = hipGetDevice(&current);
    if (e != hipSuccess) return e;
    if (current != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (current != device) {
      const hipError_t e2 = hipSetDevice(current);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    table[device] = ptr;
  }
  *addr = table[device];
  return hipSuccess;
}

// An entry (query at position t of sequence s, selected logical block b) is
// attended iff b is causal for t and the block table names a cached block.
__device__ __forceinline__ bool entry_valid(const Problem& p, int s, int b, int t) {
  if (b < 0 || b > (t >> 7)) return false;
  const int phys = p.block_table[(int64_t)s * p.max_blocks_per_seq + b];
  return phys >= 0 && phys < p.num_blocks;
}

// ------------------------------------------------------- selection inversion

struct CsrArgs {
  Problem p;
  const int32_t* sel;
  int32_t* cnt_mat;   // [num_seqs][hkv][csr_chunks][mbps]
  int32_t* list_cnt;  // [n_lists], list = (s * hkv + g) * mbps + b
  int32_t* off;
  int32_t* coff;
  int32_t* chunk_list;
  int32_t* entries;   // list order: (R << 4) | slot
  int32_t* entry_of;  // [R * 16 + slot] -> position in entries, -1 for a slot that is not attended
  int64_t n_lists;
  int csr_chunks;
  int hkv_shift;
  int chunk;
};

// Per (row chunk, group, sequence): histogram of the chunk's selected blocks
// in LDS.  Count pass: write the histogram row of the count matrix.  Fill pass
// (after the scans): turn it into write positions and scatter the entries.
template <bool FILL>
__global__ __launch_bounds__(256) void csr_chunk_kernel(CsrArgs a) {
  extern __shared__ int32_t hist[];  // [mbps] counts, then [mbps] bytes: block b maps to a cached block
  const Problem& p = a.p;
  const int k = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int mbps = p.max_blocks_per_seq;
  const int row0 = p.cu_q[s];
  const int nq = p.cu_q[s + 1] - row0;
  const int seq_len = p.seq_lens[s];
  const int first_pos = seq_len - nq;
  const int i0 = k * kCsrRows;
  const int nrows = max(0, min(nq - i0, kCsrRows));
  const int64_t list0 = ((int64_t)s * p.hkv + g) * mbps;
  int32_t* mat = a.cnt_mat + (((int64_t)s * p.hkv + g) * a.csr_chunks + k) * mbps;
  // The sequence's block table, read once: entry (t, b) is attended iff
  // 0 <= b <= t/128 and block b maps to a cached block (entry_valid).
  uint8_t* mapped = reinterpret_cast<uint8_t*>(hist + mbps);
  const int32_t* table = p.block_table + (int64_t)s * mbps;
  for (int b = threadIdx.x; b < mbps; b += blockDim.x) {
    hist[b] = 0;
    const int phys = table[b];
    mapped[b] = phys >= 0 && phys < p.num_blocks;
  }
  __syncthreads();
  auto valid = [&](int b, int t) { return b >= 0 && b <= (t >> 7) && mapped[b]; };  // t < seq_len <= mbps * 128
  // The chunk's (row, slot) entries, kU per thread requested together
  // (clamped to the last entry, so the loads issue as one batch).
  constexpr int kU = 8;
  const int n_items = nrows * kTopK;
  const int stride = (int)blockDim.x;
  auto load_batch = [&](int base, int (&bb)[kU]) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int idx = min(base + u * stride, n_items - 1);
      const int64_t R = ((int64_t)(row0 + i0 + (idx >> 4)) << a.hkv_shift) + g;
      bb[u] = a.sel[R * kTopK + (idx & 15)];
    }
  };
  for (int base = threadIdx.x; base < n_items; base += stride * kU) {
    int bb[kU];
    load_batch(base, bb);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int idx = base + u * stride;
      if (idx < n_items && valid(bb[u], first_pos + i0 + (idx >> 4))) atomicAdd(&hist[bb[u]], 1);
    }
  }
  __syncthreads();
  if (!FILL) {
    for (int b = threadIdx.x; b < mbps; b += blockDim.x) mat[b] = hist[b];
    return;
  }
  for (int b = threadIdx.x; b < mbps; b += blockDim.x) hist[b] = a.off[list0 + b] + mat[b];
  __syncthreads();
  for (int base = threadIdx.x; base < n_items; base += stride * kU) {
    int bb[kU];
    load_batch(base, bb);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int idx = base + u * stride;
      if (idx >= n_items) continue;
      const int i = i0 + (idx >> 4), slot = idx & 15;
      const int64_t R = ((int64_t)(row0 + i) << a.hkv_shift) + g;
      if (valid(bb[u], first_pos + i)) {
        const int pos = atomicAdd(&hist[bb[u]], 1);
        a.entries[pos] = (int32_t)((R << 4) | slot);
        a.entry_of[R * kTopK + slot] = pos;
      } else {
        a.entry_of[R * kTopK + slot] = -1;  // not attended: the merge skips it
      }
    }
  }
}

// Per list: exclusive prefix over the row chunks (in place) and the total.
// The column is read kU entries at a time (clamped, so the loads issue
// together) rather than one dependent load per row chunk.
__global__ __launch_bounds__(256) void csr_colscan_kernel(CsrArgs a) {
  constexpr int kU = 8;
  const int64_t list = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (list >= a.n_lists) return;
  const int mbps = a.p.max_blocks_per_seq;
  const int64_t sg = list / mbps, b = list - sg * mbps;
  int32_t* col = a.cnt_mat + sg * a.csr_chunks * mbps + b;
  int run = 0;
  for (int k0 = 0; k0 < a.csr_chunks; k0 += kU) {
    int v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = col[(int64_t)min(k0 + u, a.csr_chunks - 1) * mbps];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (k0 + u < a.csr_chunks) {
        col[(int64_t)(k0 + u) * mbps] = run;
        run += v[u];
      }
  }
  a.list_cnt[list] = run;
}

// One workgroup: exclusive scans of the list sizes (entry offsets) and of the
// per-list kvouter chunk counts (chunk offsets).  Each thread owns a run of
// consecutive lists (read kU at a time), the runs' totals are scanned within
// each wave by lane shuffles and across the 16 waves through LDS, then each
// thread writes its run's offsets.  Offsets are 32-bit, as the plan stores them.
__global__ __launch_bounds__(1024) void csr_scan_kernel(CsrArgs a) {
  constexpr int kU = 8;
  __shared__ int32_t wave_sum[2][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = a.n_lists;
  const int64_t per = (n + 1023) / 1024;
  const int64_t lo = std::min<int64_t>(n, tid * per), hi = std::min<int64_t>(n, lo + per);
  const int chunk = a.chunk;
  int32_t se = 0, sc = 0;
  for (int64_t i0 = lo; i0 < hi; i0 += kU) {
    int32_t c[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) c[u] = a.list_cnt[std::min<int64_t>(i0 + u, hi - 1)];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (i0 + u < hi) {
        se += c[u];
        sc += (c[u] + chunk - 1) / chunk;
      }
  }
  int32_t ie = se, ic = sc;  // inclusive scan over the wave's lanes
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t te = __shfl_up(ie, d), tc = __shfl_up(ic, d);
    if (lane >= d) {
      ie += te;
      ic += tc;
    }
  }
  if (lane == 63) {
    wave_sum[0][wave] = ie;
    wave_sum[1][wave] = ic;
  }
  __syncthreads();
  int32_t be = 0, bc = 0;  // the earlier waves' totals
  for (int w = 0; w < wave; ++w) {
    be += wave_sum[0][w];
    bc += wave_sum[1][w];
  }
  int32_t e = be + ie - se, c = bc + ic - sc;  // exclusive prefix of this thread's run
  for (int64_t i0 = lo; i0 < hi; i0 += kU) {
    int32_t k[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) k[u] = a.list_cnt[std::min<int64_t>(i0 + u, hi - 1)];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (i0 + u < hi) {
        a.off[i0 + u] = e;
        a.coff[i0 + u] = c;
        e += k[u];
        c += (k[u] + chunk - 1) / chunk;
      }
  }
  if (tid == 1023) {
    a.off[n] = be + ie;
    a.coff[n] = bc + ic;
  }
}

__global__ __launch_bounds__(256) void csr_chunk_map_kernel(CsrArgs a) {
  const int64_t list = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (list >= a.n_lists) return;
  for (int j = a.coff[list]; j < a.coff[list + 1]; ++j) a.chunk_list[j] = (int32_t)list;
}

// ------------------------------------------------------------- kvouter pass

struct KvOuterArgs {
  Problem p;
  const uint16_t* q;
  const int32_t* sel;
  const int32_t* entries;
  const int32_t* off;
  const int32_t* coff;
  const int32_t* chunk_list;
  // Partials, one row per (entry, head): prefill stores entry e's heads at
  // rows e*G .. e*G+G-1 (entry = position in the list order, so a workgroup
  // writes one contiguous range); decode stores (R, slot) at (R*16+slot)*G.
  uint16_t* part_o;  // fp16 [entries][G][D], natural dim order: normalised output * 2^-e
  uint16_t* out_direct;  // decode_fused_kernel: the bf16 output [total_q][hq][D]
  float* part_st;    // [entries][G][2]: (log2 of the slot's softmax mass, e)
  int64_t n_lists;
  int hkv_shift;
  int chunk;
};

// The fused decode step's second kernel: the selection is made in-kernel
// from the pooled scores (and written out), and the split path merges the
// slots of a row in the workgroup that finishes last.
struct StepArgs {
  const float* scores;  // pooled scores [total_q][hkv][ld]
  int64_t ld;
  int32_t* sel_out;     // [total_q][hkv][16]
  int32_t* counters;    // split path: finished slots per (row, group); zero on entry
};

// One (row, head) pair of a tile: where its query lives and how its keys are masked.
struct TileRow {
  bool valid;
  int64_t R;     // row * hkv + group
  int64_t prow;  // partial row: entry * G + head
  int hj;        // head within the group
  int lim;    // keys with in-block index > lim are after the query (local block only)
  const uint16_t* q;
};

// 16-byte LDS accesses at a byte offset from a base.
__device__ __forceinline__ void lds_store16(lds_byte* base, uint32_t off, u32x4 v) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(const_cast<__attribute__((address_space(3))) char*>(base + off)) = v;
}
__device__ __forceinline__ u32x4 lds_load16(lds_byte* base, uint32_t off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(base + off);
}

template <int D>
__global__ __launch_bounds__(256, 2) void kvouter_kernel(KvOuterArgs a) {
  __shared__ uint16_t k_s[kBlock * D], v_s[kBlock * D];
  __shared__ u32x4 stage_s[4 * 256];  // output staging, 4 KB per wave (two workgroups still fit a CU's 160 KB)
  const Problem& p = a.p;
  const int G = p.group;
  if ((int)blockIdx.x >= a.coff[a.n_lists]) return;
  const int list = a.chunk_list[blockIdx.x];
  const int mbps = p.max_blocks_per_seq;
  const int sg = list / mbps;
  const int b = list - sg * mbps;
  const int g = sg & ((1 << a.hkv_shift) - 1);
  const int s = sg >> a.hkv_shift;
  const int e0 = a.off[list] + ((int)blockIdx.x - a.coff[list]) * a.chunk;
  const int n_ent = min(a.chunk, a.off[list + 1] - e0);
  const int seq_len = p.seq_lens[s];
  const int row_end = p.cu_q[s + 1];
  const int phys = p.block_table[(int64_t)s * p.max_blocks_per_seq + b];
  const int64_t base = ((int64_t)phys * kBlock * p.hkv + g) * D;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  // Entry codes are requested one tile ahead with unconditional loads (a row
  // past the list end reads the last entry's code): the wait for a code then
  // leaves the block copy, the query loads and the partial stores in flight.
  const int rows = n_ent * G;
  auto code_of = [&](int tile) -> int32_t { return a.entries[e0 + min(tile * 32 + l32, rows - 1) / G]; };
  int32_t code_cur = code_of(wave), code_nxt = code_of(wave + 4);
  {  // the block's K and V into LDS, asynchronously (keys past the sequence end are never attended)
    const int64_t key_stride = (int64_t)p.hkv * D;
    const DmaLane<D, 4> dl = dma_lane<D, 4>(wave, lane, key_stride);
    const int valid = min(kBlock, seq_len - b * kBlock);
    block_dma<D, 4, false>(k_s, dl, wave, p.k + base, key_stride, valid);
    block_dma<D, 4, true>(v_s, dl, wave, p.v + base, key_stride, valid);
  }
  auto tile_row = [&](int tile, int32_t code32) -> TileRow {
    TileRow tr;
    const int rr = tile * 32 + l32;
    tr.valid = rr < rows;
    const int ei = tr.valid ? rr / G : 0;
    const int hj = tr.valid ? rr - ei * G : 0;
    const int64_t code = tr.valid ? (int64_t)code32 : 0;
    tr.R = code >> 4;
    tr.prow = (int64_t)(e0 + ei) * G + hj;
    const int64_t r = tr.R >> a.hkv_shift;
    const int t = seq_len - (row_end - (int)r);
    tr.lim = (tr.valid && (t >> 7) == b) ? t - b * kBlock : kBlock - 1;
    tr.q = a.q + (r * p.hq + g * G + hj) * D;
    tr.hj = hj;
    return tr;
  };

  // The first tile's rows and queries load while the block is in flight.
  int tile = wave;
  const bool has_tiles = tile * 32 < rows;
  // Unconditional, so the compiler can count the loads in flight: rows past
  // the list end (and a wave with no tiles) read a valid row's query;
  // nothing of theirs is stored.
  TileRow cur = tile_row(tile, code_cur);
  QRaw<D> raw;
  load_q_raw<D>(cur.q, raw);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's copies have landed
  __syncthreads();                // and everyone's
  if (!has_tiles) return;
  lds_byte* kb = opaque_lds(k_s);
  lds_byte* vb = opaque_lds(v_s);
  const OpLane<D> ol = op_lane<D>(lane);
  // This workgroup's partial rows (entry e0's first head on) and statistics.
  const auto out_o = buffer_rsrc(a.part_o + (int64_t)e0 * G * D, (uint32_t)(rows * D * 2));
  const auto out_st = buffer_rsrc(a.part_st + (int64_t)e0 * G * 2, (uint32_t)(rows * 8));
  // Output staging: the wave's 4 KB hold 64 dims of the tile's 32 rows (128
  // bytes a row) at a time, their 16-byte chunks XOR-swizzled by row (chunk c
  // of row r at r*128 + (c ^ (r/2 % 8))*16) so that neither the writes nor
  // the reads meet a bank twice in a group of 16 lanes.  Read back with eight
  // lanes per row, each store writes eight whole 128-byte row halves.
  lds_byte* stg = opaque_lds(reinterpret_cast<const uint16_t*>(stage_s)) + wave * 4096;
  uint32_t st_w[4], st_r[4];  // c1, c2 of an even and an odd dim tile; four row groups
#pragma unroll
  for (int c = 0; c < 4; ++c) st_w[c] = (uint32_t)(l32 * 128 + (((4 * (c >> 1) + 2 * (c & 1) + half) ^ ((l32 >> 1) & 7)) * 16));
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int row = 8 * k + (lane >> 3);
    st_r[k] = (uint32_t)(row * 128 + (((lane & 7) ^ ((row >> 1) & 7)) * 16));
  }
  const uint32_t st_g = (uint32_t)((lane >> 3) * D * 2 + (lane & 7) * 16);
  for (; tile * 32 < rows; tile += 4) {
    bf16x8 bq[D / 16];
    q_operand<D>(raw, bq);
    // Next tile's row and query loads are issued before this tile's math.
    const int nxt = tile + 4;
    TileRow next = cur;
    if (nxt * 32 < rows) {
      next = tile_row(nxt, code_nxt);
      load_q_raw<D>(next.q, raw);
    }
    code_nxt = code_of(nxt + 4);

    f32x16 sacc[4];
    tile_scores<D>(kb, ol, bq, sacc);
    if (__ballot(cur.lim < kBlock - 1) != 0) {  // local-block rows in this tile: mask keys after the query
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = t4 * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          sacc[t4][i] = key <= cur.lim ? sacc[t4][i] : -__builtin_inff();
        }
    }
    float m, l;
    softmax_rows(sacc, p.scale_log2e, m, l);
    f32x16 oacc[D / 32];
    {
      bf16x8 pb[8];
      p_operand(sacc, pb);
      tile_pv<D, false>(vb, ol, pb, oacc);
    }

    // Normalised output, scaled by 2^-e into [-1, 1] for fp16 storage; the
    // normalisation 1/l and the 2^-e scale are one multiply.
    float amax = 0.f;
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(oacc[n][i]));
    const float inv_l = 1.0f / l;
    amax = fmaxf(amax, swap_halves(amax)) * inv_l;
    const int ex = amax > 0.f ? (int)((__float_as_uint(amax) >> 23) & 0xff) - 126 : 0;
    const float f = ldexpf(inv_l, -ex);
    // Partial rows in natural dim order.  Lane (row rho, half h) holds dims
    // 32n + 8*(i/4) + 4h + (i%4) of oacc[n]; a swap across the wave halves
    // gives it dims 32n + 8h .. +7 (c1) and 32n + 16 + 8h .. +7 (c2), which go
    // to the staging rows; two dim tiles (64 dims) make one round through it.
    // Stores are unconditional buffer stores relative to this workgroup's
    // rows: a tile row past the list end is out of the resource's range, so
    // the hardware drops it.  (Branches around the stores would keep the
    // compiler from counting them, and the next tile's wait for its query
    // loads would then wait for these stores as well.)  The LDS accesses of
    // one wave complete in order, so a round's writes never overtake the
    // previous round's reads.  The partial rows and statistics are written
    // once and read once by the merge, so they are stored non-temporally:
    // they then stream past the caches instead of evicting the queries
    // (whole lines, so no partial-line merging is left to the caches).
#pragma unroll
    for (int ph = 0; ph < D / 64; ++ph) {
#pragma unroll
      for (int n2 = 0; n2 < 2; ++n2) {
        const f32x16& o = oacc[2 * ph + n2];
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = pack_f16x2(o[2 * i] * f, o[2 * i + 1] * f);
        const auto s0 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
        const auto s2 = __builtin_amdgcn_permlane32_swap(w[4], w[6], false, false);
        const auto s3 = __builtin_amdgcn_permlane32_swap(w[5], w[7], false, false);
        lds_store16(stg, st_w[2 * n2], u32x4{s0[0], s1[0], s0[1], s1[1]});
        lds_store16(stg, st_w[2 * n2 + 1], u32x4{s2[0], s3[0], s2[1], s3[1]});
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
        __builtin_amdgcn_raw_buffer_store_b128(lds_load16(stg, st_r[k]), out_o,
                                               st_g + (uint32_t)((tile * 32 + 8 * k) * D * 2 + ph * 128), 0, kLoadNT);
    }
    const u32x2 st{__float_as_uint(m + __log2f(l)), __float_as_uint((float)ex)};
    __builtin_amdgcn_raw_buffer_store_b64(st, out_st, half == 0 ? (uint32_t)((tile * 32 + l32) * 8) : 0xfffffff8u, 0, kLoadNT);
    cur = next;
  }
}

// --------------------------------------------------------- decode blocks

// Decode: one workgroup per (slot, group, sequence) attends the sequence's
// single query (the group's G heads) to one selected block.  At one query
// row per block this is a streaming read of 2 x 128 x D bf16 (HBM-bound), so
// nothing is staged in LDS: wave w owns keys [32w, 32w+32).  Scores use the
// 16x16x32 bf16 MFMA with the wave's keys on M (K rows read straight from the
// cache) and the group's heads on N (padded to 16); P.V uses vector ALU math
// with each lane owning D/64 output dims.  Output: the same partial rows as
// the prefill pass (row (R*16 + slot)*G + head, natural dim order, fp16 * 2^-e).
// 16x16x32 bf16 MFMA lane layout: A lane l holds A[l%16][8*(l/16) .. +7],
// B lane l holds B[8*(l/16) .. +7][l%16], D lane l register i holds
// D[4*(l/16) + i][l%16].
// LDS of one slot's decode attention (decode_block_partial).
template <int D, int GM>
struct DecodeBlockLds {
  float s_s[GM][kBlock];
  float red_s[4][GM][D];
  float stat_s[GM][4];
};

// One workgroup (4 waves) attends the sequence's single query (the group's G
// heads) at position t to block b (logical; it must satisfy entry_valid) and
// writes the partial rows (R*16 + slot)*G + head.
template <int D, bool COHERENT, bool NT = false>
__device__ __forceinline__ u32x4 merge_slots(uint32_t ok_mask, const int64_t (&prow)[kTopK], const uint16_t* part_o,
                                             const float* part_st, int d8);

// Device-coherent 16- and 8-byte loads and stores (gfx950 "sc1" buffer
// accesses: they reach the level every XCD reads, past any XCD's L2, so no
// cache write-back or invalidation is needed around them) of the partials
// that one kernel's workgroups exchange (the fused decode step's merge).
// Offsets are in bytes from the array's start.
constexpr int kCoherent = 16;
__device__ __forceinline__ void coherent_store16(void* base, uint32_t off, const u32x4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, buffer_rsrc(base, 0x7fffffffu), off, 0, kCoherent);
}
__device__ __forceinline__ void coherent_store8(void* base, uint32_t off, const u32x2& v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, buffer_rsrc(base, 0x7fffffffu), off, 0, kCoherent);
}
__device__ __forceinline__ u32x4 coherent_load16(const void* base, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(buffer_rsrc(base, 0x7fffffffu), off, 0, kCoherent);
}
__device__ __forceinline__ u32x2 coherent_load8(const void* base, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(buffer_rsrc(base, 0x7fffffffu), off, 0, kCoherent);
}

// COHERENT: the partials are stored with device-coherent stores (for a merge
// by another workgroup of the same kernel); the values are the same.
template <int D, int GM, bool COHERENT = false>
__device__ __forceinline__ void decode_block_partial(const KvOuterArgs& a, DecodeBlockLds<D, GM>& sh, int g,
                                                     int64_t R, int slot, int b, int t, int phys) {
  constexpr int VPL = D / 64;  // output dims per lane in P.V
  constexpr int KS = D / 32;   // MFMA k-steps
  auto& s_s = sh.s_s;
  auto& red_s = sh.red_s;
  auto& stat_s = sh.stat_s;
  const Problem& p = a.p;
  const int G = p.group;
  const int nvalid = min(kBlock, t - b * kBlock + 1);
  const int64_t key_stride = (int64_t)p.hkv * D;
  const uint16_t* kb = p.k + ((int64_t)phys * kBlock * p.hkv + g) * D;
  const uint16_t* vb = p.v + ((int64_t)phys * kBlock * p.hkv + g) * D;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q16 = lane >> 4;

  // V rows of this wave's keys (lane: dims lane*VPL ..), issued first; K and V by non-temporal loads (read once).
  uint32_t vreg[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int kk = wave * 32 + k;
    if constexpr (VPL == 2)
      vreg[k] = kk < nvalid ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(vb + kk * key_stride + lane * 2)) : 0u;
    else
      vreg[k] = kk < nvalid ? (uint32_t)__builtin_nontemporal_load(vb + kk * key_stride + lane) : 0u;
  }
  // K rows (A operand) for the wave's two 16-key tiles, and the heads' Q (B operand).
  bf16x8 ak[2][KS], bq[KS];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int key = wave * 32 + mt * 16 + l16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      ak[mt][ks] = as_bf16x8(key < nvalid ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + key * key_stride + ks * 32 + q16 * 8))
                                          : u32x4{0u, 0u, 0u, 0u});
  }
  const uint16_t* qh = a.q + ((R >> a.hkv_shift) * p.hq + g * G + l16) * D;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    bq[ks] = as_bf16x8(l16 < G ? load16(qh + ks * 32 + q16 * 8) : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[mt][ks], bq[ks], acc, 0, 0, 0);
    if (l16 < GM) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = wave * 32 + mt * 16 + q16 * 4 + i;
        if (l16 < G) s_s[l16][key] = key < nvalid ? acc[i] : -__builtin_inff();
      }
    }
  }
  __syncthreads();

  // Softmax statistics per head (wave w: heads w, w+4, ...), base 2.
  const float c = p.scale_log2e;
  for (int j = wave; j < G; j += 4) {
    const float z0 = s_s[j][lane], z1 = s_s[j][lane + 64];
    float mx = fmaxf(z0, z1);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    mx *= c;
    const float e0 = fast_exp2(fmaf(z0, c, -mx)), e1 = fast_exp2(fmaf(z1, c, -mx));
    s_s[j][lane] = e0;
    s_s[j][lane + 64] = e1;
    float l = e0 + e1;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
    if (lane == 0) {
      stat_s[j][0] = mx;
      stat_s[j][1] = l;
    }
  }
  __syncthreads();

  // P.V over this wave's keys, then the sum over the four waves.
  float o[GM][VPL];
#pragma unroll
  for (int j = 0; j < GM; ++j)
#pragma unroll
    for (int v = 0; v < VPL; ++v) o[j][v] = 0.f;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    float vv[VPL];
    if constexpr (VPL == 2) {
      vv[0] = bf16_to_f32(vreg[k] & 0xffffu);
      vv[1] = bf16_to_f32(vreg[k] >> 16);
    } else {
      vv[0] = bf16_to_f32(vreg[k] & 0xffffu);
    }
#pragma unroll
    for (int j = 0; j < GM; ++j) {
      const float pj = s_s[j][wave * 32 + k];
#pragma unroll
      for (int v = 0; v < VPL; ++v) o[j][v] = fmaf(pj, vv[v], o[j][v]);
    }
  }
#pragma unroll
  for (int j = 0; j < GM; ++j)
#pragma unroll
    for (int v = 0; v < VPL; ++v) red_s[wave][j][lane * VPL + v] = o[j][v];
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 256) {
    const int j = idx / D, d = idx - j * D;
    red_s[0][j][d] = (red_s[0][j][d] + red_s[1][j][d] + red_s[2][j][d] + red_s[3][j][d]) / stat_s[j][1];
  }
  __syncthreads();
  for (int j = wave; j < G; j += 4) {
    float amax = 0.f;
    for (int d = lane; d < D; d += 64) amax = fmaxf(amax, fabsf(red_s[0][j][d]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if (lane == 0) stat_s[j][2] = amax > 0.f ? (float)((int)((__float_as_uint(amax) >> 23) & 0xff) - 126) : 0.f;
  }
  __syncthreads();
  // Partial rows in natural dim order, 8 dims per store.
  for (int idx = tid; idx < G * (D / 8); idx += 256) {
    const int j = idx / (D / 8), p8 = idx - j * (D / 8);
    const float f = ldexpf(1.0f, -(int)stat_s[j][2]);
    const float* x = &red_s[0][j][p8 * 8];
    const u32x4 w{pack_f16x2(x[0] * f, x[1] * f), pack_f16x2(x[2] * f, x[3] * f), pack_f16x2(x[4] * f, x[5] * f),
                  pack_f16x2(x[6] * f, x[7] * f)};
    const int64_t prow = (R * kTopK + slot) * G + j;
    if constexpr (COHERENT)
      coherent_store16(a.part_o, (uint32_t)((prow * D + p8 * 8) * 2), w);
    else
      store16(a.part_o + prow * D + p8 * 8, w);
  }
  if (tid < G) {
    const int64_t prow = (R * kTopK + slot) * G + tid;
    const f32x2 st{stat_s[tid][0] + __log2f(stat_s[tid][1]), stat_s[tid][2]};
    if constexpr (COHERENT) {
      coherent_store8(a.part_st, (uint32_t)(prow * 8), u32x2{__float_as_uint(st[0]), __float_as_uint(st[1])});
    } else {
      *reinterpret_cast<f32x2*>(a.part_st + prow * 2) = st;
    }
  }
}

template <int D, int GM>
__global__ __launch_bounds__(256) void decode_block_kernel(KvOuterArgs a) {
  __shared__ DecodeBlockLds<D, GM> sh;
  const Problem& p = a.p;
  const int slot = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int64_t R = ((int64_t)p.cu_q[s] << a.hkv_shift) + g;
  const int b = a.sel[R * kTopK + slot];
  const int t = p.seq_lens[s] - 1;
  if (b < 0 || b > (t >> 7)) return;
  const int phys = p.block_table[(int64_t)s * p.max_blocks_per_seq + b];
  if (!(phys >= 0 && phys < p.num_blocks)) return;  // entry_valid
  decode_block_partial<D, GM>(a, sh, g, R, slot, b, t, phys);
}


// The fused decode step, small batches: one workgroup per (slot, group,
// sequence), as decode_block_kernel, that first makes its row's selection
// from the pooled scores (every slot's workgroup computes the same one with
// split_select_row, the msa_block_topk rule; slot 0's writes it out), then
// attends its slot's block.  While the scores load, the sequence's block
// table row is loaded into LDS (rows of up to kStepTab blocks), so the
// selected blocks' cache addresses and validity need no further round trip to
// memory.  The row's 16 workgroups count themselves on a per-row counter; the
// last one merges the 16 slots exactly as merge_kernel does and sets the
// counter back to 0.  The partials are exchanged through device-coherent
// stores and loads, so the merge sees every workgroup's partial whichever XCD
// wrote it.
constexpr int kStepTab = 8192;  // block-table entries staged in LDS (1M tokens)

template <int D, int GM>
__global__ __launch_bounds__(256) void decode_step_block_kernel(KvOuterArgs a, StepArgs sa) {
  constexpr int C8 = D / 8;
  constexpr int TV = kStepTab / 256;  // table entries per thread
  __shared__ union {
    int32_t tab[kStepTab];       // selection phase: the sequence's block table row
    DecodeBlockLds<D, GM> attn;  // attention phase
  } lds;
  __shared__ uint32_t surv_key[4][64];
  __shared__ int32_t surv_idx[4][64];
  __shared__ int32_t cand[4][kKeep];
  __shared__ uint32_t cand_key[4][kKeep];
  __shared__ int32_t sel_s[kTopK];
  __shared__ int32_t phys_s[kTopK];
  __shared__ uint32_t ok_s;
  __shared__ int last_s;
  const Problem& p = a.p;
  const int G = p.group;
  const int slot = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int r = p.cu_q[s];
  const int64_t R = ((int64_t)r << a.hkv_shift) + g;
  const int t = p.seq_lens[s] - 1;
  const int c = t >> 7;
  const int tid = threadIdx.x;
  const int32_t* table = p.block_table + (int64_t)s * p.max_blocks_per_seq;
  const bool tab_lds = c < kStepTab;
  int32_t tv[TV];
  if (tab_lds) {  // requested before the scores, consumed after the selection
#pragma unroll
    for (int j = 0; j < TV; ++j) tv[j] = j * 256 + tid <= c ? table[j * 256 + tid] : -1;
  }
  if (c + 1 <= kTopK) {
    if (tid < kTopK) sel_s[tid] = tid <= c ? tid : -1;
  } else {
    // <= 2048 candidates per wave in registers
    split_select_row<4, 32>(sa.scores + R * sa.ld, c, sel_s, surv_key, surv_idx, cand, cand_key);
    if (tid == 0) sel_s[kKeep] = c;
  }
  if (tab_lds) {
#pragma unroll
    for (int j = 0; j < TV; ++j)
      if (j * 256 + tid <= c) lds.tab[j * 256 + tid] = tv[j];
  }
  __syncthreads();
  if (tid < 64) {  // wave 0: each slot's cache block and whether it is attended (entry_valid)
    const int bj = tid < kTopK ? sel_s[tid] : -1;
    const bool causal = bj >= 0 && bj <= c;
    const int phys = causal ? (tab_lds ? lds.tab[bj] : table[bj]) : -1;
    const bool ok = causal && phys >= 0 && phys < p.num_blocks;
    const uint64_t m = __ballot(ok);
    if (tid < kTopK) phys_s[tid] = phys;
    if (tid == 0) ok_s = (uint32_t)m;
  }
  __syncthreads();  // (the table's LDS is free from here on)
  if (slot == 0 && tid < kTopK) sa.sel_out[R * kTopK + tid] = sel_s[tid];
  const uint32_t ok_mask = ok_s;
  if (ok_mask >> slot & 1u) decode_block_partial<D, GM, true>(a, lds.attn, g, R, slot, sel_s[slot], t, phys_s[slot]);

  // The partials were stored device-coherently; every wave waits until its
  // stores have completed before the row's counter is incremented, so the
  // workgroup that sees 15 finished before it reads complete partials (with
  // device-coherent loads).  No cache maintenance is needed.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    last_s = __hip_atomic_fetch_add(sa.counters + R, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == kTopK - 1;
  __syncthreads();
  if (!last_s) return;
  for (int idx = tid; idx < G * C8; idx += blockDim.x) {
    const int hj = idx / C8, d8 = idx - hj * C8;
    int64_t prow[kTopK];
#pragma unroll
    for (int j = 0; j < kTopK; ++j) prow[j] = ((ok_mask >> j & 1u) ? R * kTopK + j : 0) * G + hj;
    store16(a.out_direct + ((int64_t)r * p.hq + g * G + hj) * D + d8 * 8,
            merge_slots<D, true>(ok_mask, prow, a.part_o, a.part_st, d8));
  }
  if (tid == 0) sa.counters[R] = 0;
}

// Decode of a large batch: one workgroup of 16 waves per (sequence, group);
// wave w attends the query's G heads to the block of slot w, 32 keys at a
// time with an online softmax, and the 16 waves' (max, sum, output) triples
// are combined in LDS into the output row, so no partial rows are written.
// Scores use the 16x16x32 bf16 MFMA with keys on M (each step's K rows
// staged whole in the wave's LDS region, DecodeWave) and heads on N (padded
// to 16); P.V uses vector ALU math with each lane owning D/64 output dims and
// P broadcast from LDS.  Layout of the 16x16x32 operands as in
// decode_block_kernel.
template <int D, int GM>
__global__ __launch_bounds__(1024) void decode_fused_kernel(KvOuterArgs a) {
  using W = DecodeWave<D, GM>;
  __shared__ float p_s[kTopK][GM][W::SUB];
  __shared__ float alpha_s[kTopK][GM];
  __shared__ float m_s[kTopK][GM], l_s[kTopK][GM];
  __shared__ __attribute__((aligned(16))) float o_s[kTopK][GM][D];
  // Each wave's K staging: inside its own o_s rows when they are large
  // enough (they are written only after the wave's last step), else apart.
  constexpr bool kStageInOut = GM * D * 4 >= W::STAGE * 2;
  __shared__ __attribute__((aligned(16))) uint16_t kst_s[kStageInOut ? 1 : kTopK][kStageInOut ? 1 : W::STAGE];
  const Problem& p = a.p;
  const int G = p.group;
  const int g = blockIdx.x & ((1 << a.hkv_shift) - 1);
  const int s = blockIdx.x >> a.hkv_shift;
  const int r = p.cu_q[s];
  const int64_t R = ((int64_t)r << a.hkv_shift) + g;
  const int t = p.seq_lens[s] - 1;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = a.sel[R * kTopK + w];
  W st;
  if (entry_valid(p, s, b, t)) {
    const int phys = p.block_table[(int64_t)s * p.max_blocks_per_seq + b];
    bf16x8 bq[W::KS];
    st.load_q(a.q + ((int64_t)r * p.hq + g * G) * D, G, bq);
    uint16_t* stage = kStageInOut ? reinterpret_cast<uint16_t*>(&o_s[w][0][0]) : &kst_s[kStageInOut ? 0 : w][0];
    st.attend_block(p.k, p.v, ((int64_t)phys * kBlock * p.hkv + g) * D, (int64_t)p.hkv * D,
                    min(kBlock, t - b * kBlock + 1), bq, p.scale_log2e, p_s[w], alpha_s[w], stage);
  }
  st.store(o_s[w], m_s[w], l_s[w]);
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * (D / 2); idx += blockDim.x) {
    const int j = idx / (D / 2), d = (idx - j * (D / 2)) * 2;
    float o0, o1, L, M;
    combine_waves<D, GM, kTopK>(o_s, m_s, l_s, j, d, o0, o1, L, M);
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    *reinterpret_cast<uint32_t*>(a.out_direct + ((int64_t)r * p.hq + g * G + j) * D + d) = pack_bf16x2(o0 * inv, o1 * inv);
  }
}

__device__ __forceinline__ void swap_f(float& x, float& y) {
  const float t = x;
  x = y;
  y = t;
}

// Decode of a batch with fewer (sequence, group) pairs than the chip has CUs
// (but enough for one workgroup each to pay): two 16-wave workgroups per
// pair, each attending 8 of the 16 selected blocks with two waves per block
// (64 keys each), so every CU streams about half as much.  Each workgroup
// combines its waves in LDS as decode_fused_kernel does, stores its half's
// (max, mass, unnormalised output) device-coherently in the workspace, and
// counts itself on the pair's counter (zero on entry: the decode step's
// scoring kernel clears it, or a fill kernel before the decode call); the
// second to arrive reads the other half with device-coherent loads, combines
// the two in half order, writes the bf16 output and clears the counter.  One
// thread per (head, dim pair) item in both phases.
template <int D, int GM>
__global__ __launch_bounds__(1024) void decode_fused_half_kernel(KvOuterArgs a, StepArgs sa) {
  using W = DecodeWave<D, GM>;
  __shared__ float p_s[kTopK][GM][W::SUB];
  __shared__ float alpha_s[kTopK][GM];
  __shared__ float m_s[kTopK][GM], l_s[kTopK][GM];
  __shared__ __attribute__((aligned(16))) float o_s[kTopK][GM][D];
  constexpr bool kStageInOut = GM * D * 4 >= W::STAGE * 2;
  __shared__ __attribute__((aligned(16))) uint16_t kst_s[kStageInOut ? 1 : kTopK][kStageInOut ? 1 : W::STAGE];
  __shared__ int last_s;
  const Problem& p = a.p;
  const int G = p.group;
  const int half = blockIdx.x & 1;
  const int pair = blockIdx.x >> 1;
  const int g = pair & ((1 << a.hkv_shift) - 1);
  const int s = pair >> a.hkv_shift;
  const int r = p.cu_q[s];
  const int64_t R = ((int64_t)r << a.hkv_shift) + g;
  const int t = p.seq_lens[s] - 1;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = half * (kTopK / 2) + (w >> 1);
  const int k_lo = (w & 1) * (kBlock / 2);  // this wave's half of the block's keys
  const int b = a.sel[R * kTopK + slot];
  W st;
  if (entry_valid(p, s, b, t)) {
    const int nvalid = min(kBlock, t - b * kBlock + 1) - k_lo;
    if (nvalid > 0) {
      const int phys = p.block_table[(int64_t)s * p.max_blocks_per_seq + b];
      bf16x8 bq[W::KS];
      st.load_q(a.q + ((int64_t)r * p.hq + g * G) * D, G, bq);
      uint16_t* stage = kStageInOut ? reinterpret_cast<uint16_t*>(&o_s[w][0][0]) : &kst_s[kStageInOut ? 0 : w][0];
      st.attend_block(p.k, p.v, ((int64_t)phys * kBlock * p.hkv + g) * D + (int64_t)k_lo * p.hkv * D,
                      (int64_t)p.hkv * D, min(nvalid, kBlock / 2), bq, p.scale_log2e, p_s[w], alpha_s[w], stage);
    }
  }
  st.store(o_s[w], m_s[w], l_s[w]);
  __syncthreads();
  // This half's state in the step workspace: per (pair, half), G x D output
  // sums, then (max, mass) per head.
  const int stride = G * D + 2 * G;
  float* const mine = reinterpret_cast<float*>(a.part_o) + (R * 2 + half) * stride;
  const float* const other = reinterpret_cast<const float*>(a.part_o) + (R * 2 + (half ^ 1)) * stride;
  const int idx = threadIdx.x;  // G * D / 2 <= 1024 items, one per thread
  const bool item = idx < G * (D / 2);
  const int j = item ? idx / (D / 2) : 0, d = item ? (idx - j * (D / 2)) * 2 : 0;
  float o0 = 0.f, o1 = 0.f, L = 0.f, M = -__builtin_inff();
  if (item) {
    combine_waves<D, GM, kTopK>(o_s, m_s, l_s, j, d, o0, o1, L, M);
    coherent_store8(mine, (uint32_t)((j * D + d) * 4), u32x2{__float_as_uint(o0), __float_as_uint(o1)});
    if (d == 0) coherent_store8(mine, (uint32_t)((G * D + 2 * j) * 4), u32x2{__float_as_uint(M), __float_as_uint(L)});
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
  __syncthreads();                // and every thread's, before the pair's counter is incremented
  if (threadIdx.x == 0)
    last_s = __hip_atomic_fetch_add(sa.counters + R, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 1;
  __syncthreads();
  if (!last_s) return;
  if (item) {
    const u32x2 ov = coherent_load8(other, (uint32_t)((j * D + d) * 4));
    const u32x2 ml = coherent_load8(other, (uint32_t)((G * D + 2 * j) * 4));
    // Combine in half order, whichever half arrived last, so the rounding
    // (fused multiply-adds included) does not depend on the arrival order.
    float ao0 = o0, ao1 = o1, aL = L, aM = M;
    float bo0 = __uint_as_float(ov[0]), bo1 = __uint_as_float(ov[1]), bL = __uint_as_float(ml[1]),
          bM = __uint_as_float(ml[0]);
    if (half) {
      swap_f(ao0, bo0);
      swap_f(ao1, bo1);
      swap_f(aL, bL);
      swap_f(aM, bM);
    }
    const float Mx = fmaxf(aM, bM);
    const float fa = aL > 0.f ? fast_exp2(aM - Mx) : 0.f;
    const float fb = bL > 0.f ? fast_exp2(bM - Mx) : 0.f;
    const float Lt = aL * fa + bL * fb;
    const float inv = Lt > 0.f ? 1.0f / Lt : 0.f;  // no attended key: 0
    const float y0 = (ao0 * fa + bo0 * fb) * inv, y1 = (ao1 * fa + bo1 * fb) * inv;
    *reinterpret_cast<uint32_t*>(a.out_direct + ((int64_t)r * p.hq + g * G + j) * D + d) = pack_bf16x2(y0, y1);
  }
  if (threadIdx.x == 0) sa.counters[R] = 0;
}

// ----------------------------------------------------------------- merge

struct MergeArgs {
  Problem p;
  const int32_t* sel;
  const int32_t* entry_of;  // merge_prefill_kernel: partial entry of (R, slot), -1 if not attended; merge_kernel (decode): unused
  const uint16_t* part_o;
  const float* part_st;
  uint16_t* out;
  int hkv_shift;
};

// Log-sum-exp combination of one (row, head)'s attended slots for 8
// consecutive output dims d8*8 .. +7: slot j (bit j of ok_mask) holds the
// partial row prow[j] (normalised output * 2^-e, fp16) and its statistics
// (log2 of the slot's softmax mass, e).  Returns the 8 outputs as bf16.  All
// loads of the 16 slots are issued before any arithmetic.
template <int D, bool COHERENT = false, bool NT>
__device__ __forceinline__ u32x4 merge_slots(uint32_t ok_mask, const int64_t (&prow)[kTopK], const uint16_t* part_o,
                                             const float* part_st, int d8) {
  // Slot j's weight is its softmax mass 2^lse_j relative to the largest.
  float M = -__builtin_inff();
  f32x2 sj[kTopK];
  u32x4 yc[COHERENT ? kTopK : 1];
  if constexpr (COHERENT) {  // every slot's statistics and partial row in flight at once
#pragma unroll
    for (int j = 0; j < kTopK; ++j) {
      const bool ok = ok_mask >> j & 1u;
      const int64_t pr = ok ? prow[j] : 0;
      const u32x2 st = coherent_load8(part_st, (uint32_t)(pr * 8));
      sj[j] = f32x2{__uint_as_float(st[0]), __uint_as_float(st[1])};
      yc[j] = coherent_load16(part_o, (uint32_t)((pr * D + d8 * 8) * 2));
    }
#pragma unroll
    for (int j = 0; j < kTopK; ++j) {
      if (!(ok_mask >> j & 1u)) {
        sj[j] = f32x2{-__builtin_inff(), 0.f};
        yc[j] = u32x4{0u, 0u, 0u, 0u};
      }
      M = fmaxf(M, sj[j][0]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kTopK; ++j) {
      sj[j] = (ok_mask >> j & 1u) ? *reinterpret_cast<const f32x2*>(part_st + prow[j] * 2)
                                  : f32x2{-__builtin_inff(), 0.f};
      M = fmaxf(M, sj[j][0]);
    }
  }
  float L = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h8 = 0; h8 < kTopK; h8 += 8) {
    __builtin_amdgcn_sched_barrier(0);  // eight slots' loads in flight at a time
    u32x4 y[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = h8 + jj;
      if constexpr (COHERENT)
        y[jj] = yc[j];
      else
        if (!(ok_mask >> j & 1u))
        y[jj] = u32x4{0u, 0u, 0u, 0u};
      else if constexpr (NT)
        y[jj] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(part_o + prow[j] * D + d8 * 8));
      else
        y[jj] = load16(part_o + prow[j] * D + d8 * 8);
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = h8 + jj;
      const float w = (ok_mask >> j & 1u) ? fast_exp2(sj[j][0] - M) : 0.f;
      L += w;
      const float wy = ldexpf(w, (int)sj[j][1]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += wy * f16_lo(y[jj][i]);
        acc[2 * i + 1] += wy * f16_hi(y[jj][i]);
      }
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;  // no attended key (every selected block unmapped): 0
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  return o;
}

// Decode (the split path): one thread per (row, head, 8 consecutive output
// dims): log-sum-exp over the row's attended slots, then the bf16 output.  A
// slot is attended iff its block id is causal (0 <= b <= c) and the block
// table maps it to a cached block (entry_valid); decode_block_kernel wrote
// partial rows (R*16 + slot)*G + head for exactly those.  The partial rows
// are read once, by non-temporal loads.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int C8 = D / 8;
  const Problem& p = a.p;
  const int G = p.group;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = ((int64_t)p.total_q << a.hkv_shift) * G * C8;
  if (idx >= n) return;
  const int d8 = (int)(idx % C8);
  const int64_t rest = idx / C8;
  const int hj = (int)(rest % G);
  const int64_t R = rest / G;
  const int r = (int)(R >> a.hkv_shift);
  const int g = (int)(R & ((1 << a.hkv_shift) - 1));
  const int s = seq_of_row(p.cu_q, p.num_seqs, r);
  const int c = (p.seq_lens[s] - (p.cu_q[s + 1] - r)) >> 7;

  // Partial rows of the attended slots (0 for slots that are not attended).
  uint32_t ok_mask = 0;
  int64_t prow[kTopK];
#pragma unroll
  for (int j4 = 0; j4 < kTopK / 4; ++j4) {
    const u32x4 bv = load16(a.sel + R * kTopK + j4 * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j4 * 4 + i;
      const int bj = (int)bv[i];
      bool ok = bj >= 0 && bj <= c;
      if (ok) {
        const int phys = p.block_table[(int64_t)s * p.max_blocks_per_seq + bj];
        ok = phys >= 0 && phys < p.num_blocks;
      }
      ok_mask |= (ok ? 1u : 0u) << j;
      prow[j] = (ok ? R * kTopK + j : 0) * G + hj;
    }
  }
  store16(a.out + ((int64_t)r * p.hq + g * G + hj) * D + d8 * 8, merge_slots<D, false, true>(ok_mask, prow, a.part_o, a.part_st, d8));
}

// Prefill merge: one thread per (row, head, 8 consecutive output dims), as
// merge_kernel, but the plan's entry_of alone says which slots were attended
// (-1 otherwise) and where their partial rows are, so no block ids, sequence
// or block table are read.  The statistics and partial rows of all 16 slots
// are requested with unconditional loads before any arithmetic (a slot that
// was not attended reads partial row `head` of the region, which always
// exists, and its values are discarded), so each thread waits for memory
// once.  Returns the same outputs as merge_slots, slot by slot in order.
template <int D>
__global__ __launch_bounds__(256) void merge_prefill_kernel(MergeArgs a) {
  constexpr int C8 = D / 8;  // a power of two
  const Problem& p = a.p;
  const int G = p.group;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = ((int64_t)p.total_q << a.hkv_shift) * G * C8;
  if (idx >= n) return;
  // (row, head) pairs number total_q * hq < 2^31 (the output holds D values for each).
  const int d8 = (int)(idx & (C8 - 1));
  const int rest = (int)(idx / C8);
  const int R = rest / G;
  const int hj = rest - R * G;
  const int r = R >> a.hkv_shift;
  const int g = R & ((1 << a.hkv_shift) - 1);

  int32_t ent[kTopK];
#pragma unroll
  for (int j4 = 0; j4 < kTopK / 4; ++j4) {
    const u32x4 ev = load16(a.entry_of + (int64_t)R * kTopK + j4 * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) ent[j4 * 4 + i] = (int32_t)ev[i];
  }
  f32x2 st[kTopK];
  u32x4 y[kTopK];
#pragma unroll
  for (int j = 0; j < kTopK; ++j) {
    const int64_t pr = (int64_t)max(ent[j], 0) * G + hj;
    st[j] = *reinterpret_cast<const f32x2*>(a.part_st + pr * 2);
    y[j] = load16(a.part_o + pr * D + d8 * 8);
  }
  float M = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < kTopK; ++j) M = ent[j] >= 0 ? fmaxf(M, st[j][0]) : M;
  float L = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kTopK; ++j) {
    const bool ok = ent[j] >= 0;
    const float w = ok ? fast_exp2(st[j][0] - M) : 0.f;
    L += w;
    const float wy = ldexpf(w, ok ? (int)st[j][1] : 0);
    const u32x4 v = ok ? y[j] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += wy * f16_lo(v[i]);
      acc[2 * i + 1] += wy * f16_hi(v[i]);
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;  // no attended key (every selected block unmapped): 0
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  store16(a.out + ((int64_t)r * p.hq + g * G + hj) * D + d8 * 8, o);
}

// ------------------------------------------------------------------ launch

// Selection inversion into the plan region: per (sequence, group, block) lists
// of the (row, slot) entries that selected the block, and the kvouter chunks.
static hipError_t launch_plan(const Problem& p, const int32_t* sel, void* plan, hipStream_t stream) {
  const MainWs w = main_layout(p, false);
  char* base = static_cast<char*>(plan);
  CsrArgs c{p, sel,
            reinterpret_cast<int32_t*>(base + w.cnt_mat), reinterpret_cast<int32_t*>(base + w.list_cnt),
            reinterpret_cast<int32_t*>(base + w.off), reinterpret_cast<int32_t*>(base + w.coff),
            reinterpret_cast<int32_t*>(base + w.chunk_list), reinterpret_cast<int32_t*>(base + w.entries),
            reinterpret_cast<int32_t*>(base + w.entry_of), w.n_lists, w.csr_chunks, hkv_shift_of(p), w.chunk};
  const dim3 cgrid(w.csr_chunks, p.hkv, p.num_seqs);
  const size_t lds = sizeof(int32_t) * p.max_blocks_per_seq + ((p.max_blocks_per_seq + 3) & ~3);
  const unsigned list_blocks = (unsigned)((w.n_lists + 255) / 256);
  hipLaunchKernelGGL((csr_chunk_kernel<false>), cgrid, dim3(256), lds, stream, c);
  hipLaunchKernelGGL(csr_colscan_kernel, dim3(list_blocks), dim3(256), 0, stream, c);
  hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(1024), 0, stream, c);
  hipLaunchKernelGGL((csr_chunk_kernel<true>), cgrid, dim3(256), lds, stream, c);
  hipLaunchKernelGGL(csr_chunk_map_kernel, dim3(list_blocks), dim3(256), 0, stream, c);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_merge_t(const Problem& p, const int32_t* sel, const int32_t* entry_of, const uint16_t* part_o,
                                 const float* part_st, uint16_t* out, hipStream_t stream) {
  const int hs = hkv_shift_of(p);
  MergeArgs m{p, sel, entry_of, part_o, part_st, out, hs};
  const int64_t threads = ((int64_t)p.total_q << hs) * p.group * (D / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (entry_of)  // prefill
    hipLaunchKernelGGL((merge_prefill_kernel<D>), grid, dim3(256), 0, stream, m);
  else
    hipLaunchKernelGGL((merge_kernel<D>), grid, dim3(256), 0, stream, m);
  return hipGetLastError();
}

// kvouter over a computed plan, then the merge.
template <int D>
static hipError_t launch_run_t(const Problem& p, const uint16_t* q, const int32_t* sel, const void* plan,
                               uint16_t* out, void* part, hipStream_t stream) {
  const MainWs w = main_layout(p, false);
  const char* pb = static_cast<const char*>(plan);
  char* wb = static_cast<char*>(part);
  KvOuterArgs k{p, q, sel, reinterpret_cast<const int32_t*>(pb + w.entries), reinterpret_cast<const int32_t*>(pb + w.off),
                reinterpret_cast<const int32_t*>(pb + w.coff), reinterpret_cast<const int32_t*>(pb + w.chunk_list),
                reinterpret_cast<uint16_t*>(wb + w.part_o), out, reinterpret_cast<float*>(wb + w.part_st),
                w.n_lists, hkv_shift_of(p), w.chunk};
  hipLaunchKernelGGL(kvouter_kernel<D>, dim3((unsigned)w.max_kv_chunks), dim3(256), 0, stream, k);
  return launch_merge_t<D>(p, sel, reinterpret_cast<const int32_t*>(pb + w.entry_of), k.part_o, k.part_st, out, stream);
}

__global__ void clear_counters_kernel(int32_t* counters, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) counters[i] = 0;
}

template <int D>
static hipError_t launch_half_t(const Problem& p, const KvOuterArgs& k, const StepArgs& sa, hipStream_t stream) {
  const dim3 hgrid((unsigned)((int64_t)p.num_seqs * p.hkv * 2));
  if (p.group <= 4)
    hipLaunchKernelGGL((decode_fused_half_kernel<D, 4>), hgrid, dim3(1024), 0, stream, k, sa);
  else if (p.group <= 6)
    hipLaunchKernelGGL((decode_fused_half_kernel<D, 6>), hgrid, dim3(1024), 0, stream, k, sa);
  else if (p.group <= 8)
    hipLaunchKernelGGL((decode_fused_half_kernel<D, 8>), hgrid, dim3(1024), 0, stream, k, sa);
  else
    hipLaunchKernelGGL((decode_fused_half_kernel<D, 16>), hgrid, dim3(1024), 0, stream, k, sa);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_decode_t(const Problem& p, const uint16_t* q, const int32_t* sel, uint16_t* out, void* ws,
                                  hipStream_t stream) {
  const MainWs w = main_layout(p, true);
  char* base = static_cast<char*>(ws);
  KvOuterArgs k{p, q, sel, nullptr, nullptr, nullptr, nullptr,
                reinterpret_cast<uint16_t*>(base + w.part_o), out, reinterpret_cast<float*>(base + w.part_st),
                w.n_lists, hkv_shift_of(p), w.chunk};
  if (decode_uses_half(p)) {
    // Two workgroups per pair; their counters (after the halves' state) are
    // cleared first by a small kernel, the workspace being the caller's.
    int32_t* counters = reinterpret_cast<int32_t*>(base + w.part_o + decode_half_state_bytes(p));
    const int n = p.total_q * p.hkv;
    hipLaunchKernelGGL(clear_counters_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, counters, n);
    return launch_half_t<D>(p, k, StepArgs{nullptr, 0, nullptr, counters}, stream);
  }
  if ((int64_t)p.num_seqs * p.hkv >= kFusedDecodeMinGroups) {
    // Enough (sequence, group) pairs to fill the chip: one workgroup each, no merge pass.
    const unsigned n = (unsigned)(p.num_seqs * p.hkv);
    if (p.group <= 4)
      hipLaunchKernelGGL((decode_fused_kernel<D, 4>), dim3(n), dim3(1024), 0, stream, k);
    else if (p.group <= 6)
      hipLaunchKernelGGL((decode_fused_kernel<D, 6>), dim3(n), dim3(1024), 0, stream, k);
    else if (p.group <= 8)
      hipLaunchKernelGGL((decode_fused_kernel<D, 8>), dim3(n), dim3(1024), 0, stream, k);
    else
      hipLaunchKernelGGL((decode_fused_kernel<D, 16>), dim3(n), dim3(1024), 0, stream, k);
    return hipGetLastError();
  }
  const dim3 dgrid(kTopK, p.hkv, p.num_seqs);
  if (p.group <= 4)
    hipLaunchKernelGGL((decode_block_kernel<D, 4>), dgrid, dim3(256), 0, stream, k);
  else if (p.group <= 6)
    hipLaunchKernelGGL((decode_block_kernel<D, 6>), dgrid, dim3(256), 0, stream, k);
  else if (p.group <= 8)
    hipLaunchKernelGGL((decode_block_kernel<D, 8>), dgrid, dim3(256), 0, stream, k);
  else
    hipLaunchKernelGGL((decode_block_kernel<D, 16>), dgrid, dim3(256), 0, stream, k);
  return launch_merge_t<D>(p, sel, nullptr, k.part_o, k.part_st, out, stream);
}

hipError_t launch_attn_prefill_plan(const Problem& p, const int32_t* sel, void* plan, hipStream_t stream) {
  if (p.total_q == 0) return hipSuccess;
  return launch_plan(p, sel, plan, stream);
}

hipError_t launch_attn_prefill_run(const Problem& p, const uint16_t* q, const int32_t* sel, const void* plan,
                                   uint16_t* out, void* part, hipStream_t stream) {
  if (p.total_q == 0) return hipSuccess;
  return p.head_dim == 128 ? launch_run_t<128>(p, q, sel, plan, out, part, stream)
                           : launch_run_t<64>(p, q, sel, plan, out, part, stream);
}

hipError_t launch_attn_prefill(const Problem& p, const uint16_t* q, const int32_t* sel, uint16_t* out, void* ws,
                               hipStream_t stream) {
  if (p.total_q == 0) return hipSuccess;
  const hipError_t e = launch_plan(p, sel, ws, stream);
  if (e != hipSuccess) return e;
  return launch_attn_prefill_run(p, q, sel, ws, out, static_cast<char*>(ws) + prefill_plan_bytes(p), stream);
}

hipError_t launch_attn_decode(const Problem& p, const uint16_t* q, const int32_t* sel, uint16_t* out, void* ws,
                              hipStream_t stream) {
  if (p.total_q == 0) return hipSuccess;
  return p.head_dim == 128 ? launch_decode_t<128>(p, q, sel, out, ws, stream)
                           : launch_decode_t<64>(p, q, sel, out, ws, stream);
}

// ------------------------------------------------------- fused decode step

// Workspace of the fused decode step: the split decode's partial rows, then
// one counter per (row, group).
size_t decode_step_workspace_bytes(const Problem& p) {
  return decode_workspace_bytes(p) + align256(sizeof(int32_t) * (size_t)p.total_q * p.hkv);
}

int32_t* decode_step_counters(const Problem& p, void* ws) {
  if ((int64_t)p.num_seqs * p.hkv >= kFusedHalfMaxGroups) return nullptr;  // one workgroup per pair merges in LDS
  return reinterpret_cast<int32_t*>(static_cast<char*>(ws) + decode_workspace_bytes(p));
}

template <int D>
static hipError_t launch_step_attn_t(const Problem& p, const uint16_t* q, const float* scores, int64_t ld,
                                     int32_t* sel, uint16_t* out, void* ws, int64_t max_blocks, hipStream_t stream) {
  const MainWs w = main_layout(p, true);
  char* base = static_cast<char*>(ws);
  KvOuterArgs k{p, q, sel, nullptr, nullptr, nullptr, nullptr,
                reinterpret_cast<uint16_t*>(base + w.part_o), out, reinterpret_cast<float*>(base + w.part_st),
                w.n_lists, hkv_shift_of(p), w.chunk};
  const StepArgs sa{scores, ld, sel, decode_step_counters(p, ws)};
  const int64_t pairs = (int64_t)p.num_seqs * p.hkv;
  if (pairs >= kFusedDecodeMinGroups) {
    // Batches that fill the chip with one or two workgroups per (sequence,
    // group): the selection as its own short kernel (made inside each
    // workgroup, it would delay every workgroup's attention by its latency),
    // then the attention.
    const hipError_t e = launch_block_topk(p, scores, ld, sel, max_blocks, stream);
    if (e != hipSuccess) return e;
    if (pairs >= kFusedHalfMaxGroups) return launch_decode_t<D>(p, q, sel, out, ws, stream);
    return launch_half_t<D>(p, k, sa, stream);  // the step's counters, cleared by its scoring kernel
  }
  const dim3 dgrid(kTopK, p.hkv, p.num_seqs);
  if (p.group <= 4)
    hipLaunchKernelGGL((decode_step_block_kernel<D, 4>), dgrid, dim3(256), 0, stream, k, sa);
  else if (p.group <= 6)
    hipLaunchKernelGGL((decode_step_block_kernel<D, 6>), dgrid, dim3(256), 0, stream, k, sa);
  else if (p.group <= 8)
    hipLaunchKernelGGL((decode_step_block_kernel<D, 8>), dgrid, dim3(256), 0, stream, k, sa);
  else
    hipLaunchKernelGGL((decode_step_block_kernel<D, 16>), dgrid, dim3(256), 0, stream, k, sa);
  return hipGetLastError();
}

hipError_t launch_decode_step_attn(const Problem& p, const uint16_t* q, const float* scores, int64_t ld, int32_t* sel,
                                   uint16_t* out, void* ws, int64_t max_blocks, hipStream_t stream) {
  if (p.total_q == 0) return hipSuccess;
  return p.head_dim == 128 ? launch_step_attn_t<128>(p, q, scores, ld, sel, out, ws, max_blocks, stream)
                           : launch_step_attn_t<64>(p, q, scores, ld, sel, out, ws, max_blocks, stream);
}

}  // namespace msa
