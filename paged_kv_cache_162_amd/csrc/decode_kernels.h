// The paged decode attention kernels for gfx950 and their launchers, shared
// by decode.hip (entry points, split-K merge) and decode_variants.hip, which
// is compiled once per (block size, load policy) so the kernel instantiations
// build in parallel.
//
// Pages cited in this file:
//   [1] "PagedAttention - how vLLM stopped wasting 80% of your GPU memory"
//       (shivam2003.com/posts/pagedattention.html)
//   [2] "PagedAttention: How vLLM Borrowed Virtual Memory to Unlock GPU
//       Serving at Scale" (fp4-site.pages.dev/system/pagedattention-vllm-deep-dive/)
//   [3] "PagedAttention and vLLM: Virtual Memory for the KV Cache" (passgenai.com)
//   [4] "What is paged attention?" (netraruntime.com/learn/paged-attention)
//
// Pool layout per layer ([2], "The Custom CUDA Kernel"):
// [num_blocks][num_kv_heads][16][head_dim]. One (block, KV head) is a
// contiguous 16 x head_dim tile: 4 KB for 16-bit elements at head_dim 128.
//
// Decode attention computes, per sequence and query head, the softmax of the
// scaled dot products with every live key and the weighted sum of the values
// - exactly the contiguous-cache result ([1], "The PagedAttention kernel").
// Work split: one workgroup of one wave64 per (sequence, KV head, context
// partition). The partition's block-table entries are read once, one per
// lane, and broadcast from registers, so every K/V address is known before
// the first load. The wave keeps an online softmax (running max and sum, [2]
// "The Custom CUDA Kernel") over its partition. Sequences longer than one
// partition write unnormalised partial results, which a second kernel
// merges with the log-sum-exp rule.
//
// Softmax runs in base 2: scores are multiplied by scale*log2(e) and
// exponentiated with v_exp_f32; the result is the same softmax.

#ifndef PAGEDKV_DECODE_KERNELS_H_
#define PAGEDKV_DECODE_KERNELS_H_

#include "device_common.h"

namespace pagedkv {
namespace decode {

using namespace pagedkv::dev;


constexpr int kTile = 16;            // tokens per compute tile (MFMA rows / VALU block step)
constexpr int kMaxPartition = 1024;  // tokens per partition
// a partition's tiles fit one wave's lanes, so its table entries do too (one
// per lane, or two with 8-token blocks)
static_assert(kMaxPartition / kTile <= 64, "partition larger than a wave's table staging");
constexpr int kDefaultPartition = 512;
constexpr int kStageStride = 132;  // floats per head row in LDS (128 + 4 against bank conflicts)
#ifndef PAGEDKV_DECODE_RING
#define PAGEDKV_DECODE_RING 3
#endif
constexpr int kDecodeRing = PAGEDKV_DECODE_RING;  // K/V blocks in flight per wave (MFMA decode)
#ifndef PAGEDKV_DECODE_RING_PRE
#define PAGEDKV_DECODE_RING_PRE 4
#endif
// the shared-prefix step's tail units: short tails give few waves per SIMD,
// so a deeper ring pays (207 VGPRs, two waves per SIMD)
constexpr int kDecodeRingPre = PAGEDKV_DECODE_RING_PRE;
#ifndef PAGEDKV_DECODE_RING8
#define PAGEDKV_DECODE_RING8 4
#endif
// fp8 cache: a raw tile holds half the bytes, but its widened copy costs
// registers; four tiles in flight keep the kernel at three waves per SIMD
// (164 VGPRs), which measured faster than six tiles at two waves
constexpr int kDecodeRing8 = PAGEDKV_DECODE_RING8;

// ---- shared decode parameters ----------------------------------------------
struct DecodeParams {
  float* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* tables;
  const int32_t* lens;
  const int32_t* items;  // optional work plan: [n_items][2] = (sequence, partition)
  float* ws_o;           // [S][Hkv][nparts][G][D]  partial outputs (unnormalised)
  float* ws_ml;          // [S][Hkv][nparts][G][2]  partial (max, sum) in base-2 units
  // fused cache write (all NULL for a plain decode): the new token of each
  // sequence, [S][Hkv][D], is written at its last position; slots [S]
  const void* k_new;
  const void* v_new;
  void* k_pool_w;
  void* v_pool_w;
  int64_t* slots;
  // Tail mode: the first skip_tokens positions of every sequence (whole
  // blocks, shared by all of them) are left out - the kernel attends to
  // positions [skip_tokens, lens[s]) and reads the tables from entry
  // skip_tokens / block_size on; 0 otherwise.
  int32_t skip_tokens;
  // Shared-prefix step: the prefix ranges' normalised outputs
  // [pre_parts][S][Hq][D] and log2 of their softmax denominators
  // [pre_parts][S][Hq], folded into each output by the kernel that writes it
  // (pre_parts 0 otherwise).
  const float* pre_o;
  const float* pre_lse;
  int32_t pre_parts;
  int32_t max_blocks, S, Hq, Hkv, G, num_blocks, block_size, part_tokens, nparts, n_units;
  float scale_log2;  // scale * log2(e), times the K scale for an fp8 cache
  // fp8 cache: the per-pool scales (stored value = code value * scale)
  float k_scale, v_scale;
};

// Wave u of the grid (one wave per workgroup) processes work unit u: one
// (sequence, KV head, partition). With a plan, u = item * Hkv + head and the
// items are sorted longest first; since workgroups go to the eight XCDs in
// turn, a head count that is a multiple of 8 keeps every unit of one KV head
// on one XCD (and its L2). Without a plan, u enumerates (partition, head,
// sequence) over every possible partition and units past a sequence's end
// return at once.
struct WorkItem {
  int s, h, part;
  bool ok;
};
__device__ __forceinline__ WorkItem unit_item(const DecodeParams& p, int u) {
  WorkItem w;
  if (p.items) {
    const int it = u / p.Hkv;
    w.h = u % p.Hkv;
    w.s = p.items[2 * it];
    w.part = p.items[2 * it + 1];
    w.ok = w.s >= 0 && w.s < p.S && w.part >= 0 && w.part < p.nparts;
  } else {
    w.s = u % p.S;
    w.h = (u / p.S) % p.Hkv;
    w.part = u / (p.S * p.Hkv);
    w.ok = true;
  }
  return w;
}

// Shared-prefix step: the attention of output row `row` (sequence, query
// head) over the sequence's tail - v, float4 c4 of the normalised output,
// with lb = log2 of its softmax denominator, -inf for an empty tail - and
// over the prefix ranges, combined into the attention over the whole
// context:
//   out = sum_k o_k 2^(lse_k - M) / sum_k 2^(lse_k - M),  M = max_k lse_k,
// k over the ranges and the tail (softmax over a union of key sets). Every
// range's loads are issued before any is used; a NaN denominator (invalid
// sequence or table) gives NaN.
__device__ __forceinline__ float4 with_prefix(const DecodeParams& p, size_t row, int c4, int d4,
                                              float4 v, float lb) {
  constexpr int K = pagedkv::kMaxSharedParts;
  const size_t rows = (size_t)p.S * p.Hq;
  const float4* po = reinterpret_cast<const float4*>(p.pre_o);
  float la[K];
  float4 a[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    la[k] = k < p.pre_parts ? p.pre_lse[k * rows + row] : neg_inf();
    a[k] = k < p.pre_parts ? po[(k * rows + row) * d4 + c4] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float M = lb;
  bool nan = lb != lb;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    nan = nan || la[k] != la[k];
    M = fmaxf(M, la[k]);
  }
  const float wb = fast_exp2(lb - M);  // 0 for an empty tail
  float4 acc = make_float4(v.x * wb, v.y * wb, v.z * wb, v.w * wb);
  float den = wb;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const float w = fast_exp2(la[k] - M);  // 0 for the unused ranges
    acc.x += a[k].x * w;
    acc.y += a[k].y * w;
    acc.z += a[k].z * w;
    acc.w += a[k].w * w;
    den += w;
  }
  const float inv = 1.0f / den;
  const float nanf = __builtin_nanf("");
  return nan ? make_float4(nanf, nanf, nanf, nanf)
             : make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

// Sequence-level checks (one wave). Returns the number of partitions of the
// sequence when this unit has tokens to process, else 0. The output of an
// empty or invalid sequence is written here by its partition-0 unit: zeros,
// or NaN for a length that is negative or exceeds the table or
// max_context_len.
template <int D, bool PRE>
__device__ __forceinline__ int unit_prologue(const DecodeParams& p, const WorkItem& w, int ctx,
                                             int lane) {
  const bool bad = ctx < 0 ||
                   (int64_t)ctx + p.skip_tokens > (int64_t)p.max_blocks * p.block_size ||
                   (int64_t)ctx > (int64_t)p.nparts * p.part_tokens;
  if (bad || ctx == 0) {
    if (w.part == 0) {
      const float v = bad ? __builtin_nanf("") : 0.0f;
      const size_t row0 = (size_t)w.s * p.Hq + (size_t)w.h * p.G;
      float4* dst = reinterpret_cast<float4*>(p.out + row0 * D);
      for (int c = lane; c < p.G * (D / 4); c += 64) {
        float4 r = make_float4(v, v, v, v);
        // an empty tail: the prefix alone
        if constexpr (PRE) r = with_prefix(p, row0 + c / (D / 4), c % (D / 4), D / 4, r, bad ? v : neg_inf());
        dst[c] = r;
      }
      if (p.slots && w.h == 0 && lane == 0) p.slots[w.s] = -1;  // no new token to place
    }
    return 0;
  }
  const int nps = (ctx + p.part_tokens - 1) / p.part_tokens;
  return w.part < nps ? nps : 0;
}

// A partition's table entries, held by the wave that reads them ([2], "The
// Custom CUDA Kernel": the kernel resolves logical blocks through the block
// table). With blocks of 16 or 32 tokens lane i holds entry i (a partition of
// at most 64 tiles has at most 64 entries); with 8-token blocks lane i holds
// entries 2i and 2i+1, so a partition of 64 tiles (128 entries) still fits.
// Any entry j is then read by every lane with readlane. An ID outside the
// pool marks the unit invalid and is replaced by block 0, so no load leaves
// the pool; entries past the partition's end read as block 0.
struct Entries {
  int lo, hi;  // entry lane * K (and lane * K + 1 when K = 2)
};
template <int BS>
constexpr int entries_per_lane() {
  return BS < kTile ? 2 : 1;
}

// Replace out-of-pool and unused entries (index >= nent) by block 0 and
// report whether any used entry is outside the pool.
template <int BS>
__device__ __forceinline__ Entries check_entries(const DecodeParams& p, Entries raw, int nent,
                                                 int lane, bool& bad) {
  constexpr int K = entries_per_lane<BS>();
  const int i0 = lane * K;
  const bool bad0 = i0 < nent && (raw.lo < 0 || raw.lo >= p.num_blocks);
  const bool bad1 = K == 2 && i0 + 1 < nent && (raw.hi < 0 || raw.hi >= p.num_blocks);
  bad = __builtin_amdgcn_ballot_w64(bad0 || bad1) != 0;
  Entries e;
  e.lo = (bad0 || i0 >= nent) ? 0 : raw.lo;
  e.hi = (K == 1 || bad1 || i0 + 1 >= nent) ? 0 : raw.hi;
  return e;
}

// Load the partition's entries from its table row (row[0] = the partition's
// first block; at most `avail` entries exist in the row) and check them.
template <int BS>
__device__ __forceinline__ Entries stage_entries(const DecodeParams& p, const int32_t* row,
                                                 int avail, int nent, int lane, bool& bad) {
  constexpr int K = entries_per_lane<BS>();
  Entries raw{0, 0};
  if (lane * K < avail) raw.lo = row[lane * K];
  if (K == 2 && lane * K + 1 < avail) raw.hi = row[lane * K + 1];
  return check_entries<BS>(p, raw, nent, lane, bad);
}

// Entry e (wave-uniform) of the partition.
template <int BS>
__device__ __forceinline__ int entry_at(const Entries& st, int e) {
  if constexpr (BS < kTile)
    return (e & 1) ? __builtin_amdgcn_readlane(st.hi, e >> 1)
                   : __builtin_amdgcn_readlane(st.lo, e >> 1);
  else
    return __builtin_amdgcn_readlane(st.lo, e);
}

// Fused cache write ([3], "The allocation lifecycle": each decode step
// writes the new token's K,V into the last block). The unit holding the
// sequence's last position ctx-1 - the last row in use of its last block -
// owns that token's row for its KV head: it returns the row's slot
// (table[(ctx-1)/B]*B + (ctx-1)%B, [4] "How it works"), or -1 when the
// unit is invalid, and the caller stores the row before loading any block.
// No other unit reads the row.
struct NewToken {
  bool on;        // this unit places the new token
  int row;        // row of the token in the unit's last 16-token tile
  int64_t slot;   // -1 if nothing is written (invalid unit)
};
template <int BS>
__device__ __forceinline__ NewToken new_token(const DecodeParams& p, const WorkItem& w, int nps,
                                              int ctx, int t0, const Entries& staged, bool bad,
                                              int lane) {
  NewToken t;
  t.on = p.k_new != nullptr && w.part == nps - 1;
  t.row = (ctx - 1) % kTile;
  const int blk = (ctx - 1 - t0) / p.block_size;  // partition block holding ctx-1
  t.slot = (t.on && !bad) ? (int64_t)entry_at<BS>(staged, blk) * p.block_size + (ctx - 1) % p.block_size
                          : -1;
  if (t.on && p.slots && w.h == 0 && lane == 0) p.slots[w.s] = t.slot;
  return t;
}

// Index, in units of `unit` elements per token row, of row r (0..15) of
// 16-token tile j of a partition for KV head h. Blocks of 16 or 32 tokens
// hold a whole tile (one table entry per tile, wave-uniform); blocks of 8
// tokens hold half a tile, so rows 0..7 and 8..15 use consecutive entries.
template <int BS>
__device__ __forceinline__ size_t tile_row(const DecodeParams& p, int h, const Entries& staged,
                                           int j, int r, int unit) {
  int e, rb;
  if constexpr (BS >= kTile) {
    e = entry_at<BS>(staged, (kTile * j) / BS);
    rb = (kTile * j) % BS + r;
  } else {
    // entries 2j and 2j+1: both held by lane j
    const int e_lo = __builtin_amdgcn_readlane(staged.lo, j);
    const int e_hi = __builtin_amdgcn_readlane(staged.hi, j);
    e = r < 8 ? e_lo : e_hi;
    rb = r & 7;
  }
  return (((size_t)e * p.Hkv + h) * BS + rb) * unit;
}

// Start of the unit's partial results: the G heads of (sequence, KV head,
// partition) are contiguous, G x D outputs then G (max, sum) pairs.
__device__ __forceinline__ size_t partial_group(const DecodeParams& p, const WorkItem& w) {
  return ((size_t)w.s * p.Hkv + w.h) * p.nparts + w.part;
}

// Store n (multiple of 4) consecutive floats of group head g from dimension
// d0: the final output o / l for a single-partition sequence, else the
// partial o and, from the lane with write_ml, the pair (m, l). An invalid
// unit stores NaN.
template <bool PRE>
__device__ __forceinline__ void store_result(const DecodeParams& p, const WorkItem& w, int nps,
                                             int g, int d0, const float* o, int n, float m,
                                             float l, bool write_ml, bool bad, int D) {
  const float nan = __builtin_nanf("");
  if (nps == 1) {
    const size_t row = (size_t)w.s * p.Hq + (size_t)w.h * p.G + g;
    float* dst = p.out + row * D + d0;
    const float inv = 1.0f / l;
    for (int i = 0; i < n; i += 4) {
      float4 v = make_float4(o[i] * inv, o[i + 1] * inv, o[i + 2] * inv, o[i + 3] * inv);
      if (bad) v = make_float4(nan, nan, nan, nan);
      if constexpr (PRE) v = with_prefix(p, row, (d0 + i) / 4, D / 4, v, bad ? nan : m + log2f(l));
      *reinterpret_cast<float4*>(dst + i) = v;
    }
  } else {
    const size_t grp = partial_group(p, w);
    float* dst = p.ws_o + (grp * p.G + g) * D + d0;
    for (int i = 0; i < n; i += 4)
      *reinterpret_cast<float4*>(dst + i) = make_float4(o[i], o[i + 1], o[i + 2], o[i + 3]);
    if (write_ml)
      *reinterpret_cast<float2*>(p.ws_ml + (grp * p.G + g) * 2) =
          bad ? make_float2(nan, nan) : make_float2(m, l);
  }
}

// ============================================================================
// Split-K merge ([2], "The Custom CUDA Kernel": per-piece partial outputs and
// softmax denominators, merged with a numerically stable rule):
//   M = max_k m_k,  L = sum_k l_k 2^(m_k - M),  out = sum_k 2^(m_k - M) o_k / L.
// One workgroup per (sequence, KV head); sequences with one partition were
// finished by the decode kernel and return at once. Thread t merges float4
// chunk t of the group's G x D outputs with a running (online) merge in
// partition order, so for each partition the workgroup reads that
// partition's G x D partials as one contiguous span and writes the group's
// outputs as one contiguous span. A NaN partial sum (invalid table entry)
// makes the output NaN.
// ============================================================================
constexpr int kMergeThreads = 256;

template <int D, bool PRE>
__global__ __launch_bounds__(kMergeThreads) void splitk_merge_kernel(DecodeParams p) {
  const int s = blockIdx.x / p.Hkv, h = blockIdx.x % p.Hkv;
  const int ctx = p.lens[s] - p.skip_tokens;
  if (ctx <= 0 || (int64_t)ctx + p.skip_tokens > (int64_t)p.max_blocks * p.block_size ||
      (int64_t)ctx > (int64_t)p.nparts * p.part_tokens)
    return;  // written by the decode kernel
  const int nps = (ctx + p.part_tokens - 1) / p.part_tokens;
  if (nps <= 1) return;
  const size_t grp0 = ((size_t)s * p.Hkv + h) * p.nparts;  // partition 0 of the group
  const int n_chunks = p.G * (D / 4);
  for (int c = threadIdx.x; c < n_chunks; c += kMergeThreads) {
    const int g = c / (D / 4);
    const float2* ml = reinterpret_cast<const float2*>(p.ws_ml) + grp0 * p.G + g;
    const float* po = p.ws_o + grp0 * p.G * D + (size_t)c * 4;
    // running merge in partition order; the loads of eight partitions are
    // independent of the arithmetic and issue together
    float M = neg_inf(), L = 0.f;
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
    bool bad = false;
#pragma unroll 8
    for (int k = 0; k < nps; ++k) {
      const float2 v = ml[(size_t)k * p.G];
      const float4 o = *reinterpret_cast<const float4*>(po + (size_t)k * p.G * D);
      bad |= (v.y != v.y);
      const float Mn = fmaxf(M, v.x);
      const float a = fast_exp2(M - Mn);  // 0 while M is -inf
      const float b = fast_exp2(v.x - Mn);
      L = L * a + v.y * b;
      O.x = O.x * a + o.x * b;
      O.y = O.y * a + o.y * b;
      O.z = O.z * a + o.z * b;
      O.w = O.w * a + o.w * b;
      M = Mn;
    }
    const float inv = 1.0f / L;
    float4 r = make_float4(O.x * inv, O.y * inv, O.z * inv, O.w * inv);
    if (bad) r = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                             __builtin_nanf(""));
    if constexpr (PRE)
      r = with_prefix(p, (size_t)s * p.Hq + (size_t)h * p.G + g, c % (D / 4), D / 4, r,
                      bad ? __builtin_nanf("") : M + log2f(L));
    *reinterpret_cast<float4*>(p.out + ((size_t)s * p.Hq + (size_t)h * p.G) * D + (size_t)c * 4) = r;
  }
}

// ============================================================================
// Decode on the vector ALUs: any dtype, head_dim 64/128, up to GMAX query
// heads per KV head. Each token row of a block is spread over LPR lanes
// (16 bytes per lane), so one dwordx4 load per lane reads TPI whole rows and a
// 16-token block takes IPB loads. Dot products are finished with DPP row
// reductions. Each group of LPR lanes keeps its own online softmax over the
// tokens it reads; the groups are merged with cross-lane shuffles at the end.
// With an fp8 cache (KV8; DT is then the query's 16-bit type) a lane loads the
// 8 codes of the same 8 elements (8 bytes) and widens them exactly to DT; the
// K scale is folded into the score scale and the V scale into the result.
// ============================================================================
template <int DT, int D, int GMAX, int BS, bool NT, bool PRE = false, bool KV8 = false>
__global__ __launch_bounds__(64) void decode_valu_kernel(DecodeParams p) {
  constexpr int EB = DT == KV_F32 ? 4 : 2;
  constexpr int EPL = 16 / EB;           // elements per lane chunk
  constexpr int LPR = D * EB / 16;       // lanes per token row
  constexpr int TPI = 64 / LPR;          // rows per wave-wide load
  constexpr int IPB = kTile / TPI;       // loads per 16-token tile
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "unsupported row width");
  static_assert(!KV8 || (DT != KV_F32 && !PRE), "fp8 cache: 16-bit queries, plain step");
  // a lane's chunk of a pool row: 16 bytes of 16-bit/fp32 elements, or the
  // 8 codes of the same 8 elements
  typedef typename std::conditional<KV8, uint2, uint4>::type Raw;

  const int lane = threadIdx.x;
  const int u = blockIdx.x;
  if (u >= p.n_units) return;
  const int r = lane / LPR, c = lane % LPR;
  const WorkItem w = unit_item(p, u);
  if (!w.ok) return;
  const int ctx = p.lens[w.s] - p.skip_tokens;
  const int nps = unit_prologue<D, PRE>(p, w, ctx, lane);
  if (nps == 0) return;
  const int t0 = w.part * p.part_tokens;
  const int t1 = min(ctx, t0 + p.part_tokens);
  const int nblk = (t1 - t0 + kTile - 1) / kTile;        // 16-token tiles
  const int nent = (t1 - t0 + BS - 1) / BS;              // table entries (blocks)
  const int e0 = (p.skip_tokens + t0) / BS;              // the partition's first entry
  const int32_t* row = p.tables + (size_t)w.s * p.max_blocks + e0;
  bool bad = false;
  const Entries staged = stage_entries<BS>(p, row, p.max_blocks - e0, nent, lane, bad);
  const NewToken nt = new_token<BS>(p, w, nps, ctx, t0, staged, bad, lane);
  if (nt.on && nt.slot >= 0 && r == nt.row % TPI) {
    // the lanes of row group nt.row % TPI load chunk c of the new token's
    // rows with the last tile; they store those chunks first, so program
    // order within the lane makes that load return the new values
    const size_t src = ((size_t)w.s * p.Hkv + w.h) * LPR + c;
    const size_t dst = tile_row<BS>(p, w.h, staged, nblk - 1, nt.row, LPR) + c;
    const uint4 kn = static_cast<const uint4*>(p.k_new)[src];
    const uint4 vn = static_cast<const uint4*>(p.v_new)[src];
    if constexpr (KV8) {  // quantised: the 8 codes of the lane's 8 elements
      static_cast<uint2*>(p.k_pool_w)[dst] = e4m3x8_from16<DT>(kn, p.k_scale);
      static_cast<uint2*>(p.v_pool_w)[dst] = e4m3x8_from16<DT>(vn, p.v_scale);
    } else {
      static_cast<uint4*>(p.k_pool_w)[dst] = kn;
      static_cast<uint4*>(p.v_pool_w)[dst] = vn;
    }
  }

  // query chunk of every head in the group, pre-scaled into base-2 logits
  float qf[GMAX][EPL];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g < p.G) {
      const uint4* qp = reinterpret_cast<const uint4*>(
          static_cast<const char*>(p.q) + (((size_t)w.s * p.Hq + (size_t)w.h * p.G + g) * D) * EB);
      unpack16<DT>(qp[c], qf[g]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[g][e] *= p.scale_log2;
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[g][e] = 0.f;
    }
  }

  float m[GMAX], l[GMAX], acc[GMAX][EPL];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    m[g] = neg_inf();
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  const Raw* kbase = static_cast<const Raw*>(p.k_pool);
  const Raw* vbase = static_cast<const Raw*>(p.v_pool);

  // rows past the tile's live tokens read the last live row instead (their
  // values are masked), so the unused rows of a sequence's last block are
  // never fetched
  auto load = [&](int j, Raw* ku, Raw* vu) {
    const int lim = t1 - (t0 + j * kTile) - 1;  // last live row of tile j
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      const size_t at = tile_row<BS>(p, w.h, staged, j, min(r + TPI * i, lim), LPR) + c;
      ku[i] = load_kv<NT>(kbase + at);
      vu[i] = load_kv<NT>(vbase + at);
    }
  };

  auto compute = [&](int jb, const Raw* ku, const Raw* vu) {
    const int valid = t1 - (t0 + jb * kTile);  // live tokens in this tile (>= 1)
    const bool full = valid >= kTile;
    float kf[IPB][EPL], vf[IPB][EPL];
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      if constexpr (KV8) {
        unpack16<DT>(e4m3x8_widen<DT>(ku[i].x, ku[i].y), kf[i]);
        unpack16<DT>(e4m3x8_widen<DT>(vu[i].x, vu[i].y), vf[i]);
      } else {
        unpack16<DT>(ku[i], kf[i]);
        unpack16<DT>(vu[i], vf[i]);
      }
    }
    if (!full) {
#pragma unroll
      for (int i = 0; i < IPB; ++i)
        if (r + TPI * i >= valid) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) vf[i][e] = 0.f;  // masked rows may hold NaN
        }
    }
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      float sc[IPB];
#pragma unroll
      for (int i = 0; i < IPB; ++i) {
        float d0 = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) d0 = fmaf(qf[g][e], kf[i][e], d0);
        sc[i] = row_sum<LPR>(d0);
      }
      if (!full) {
#pragma unroll
        for (int i = 0; i < IPB; ++i)
          if (r + TPI * i >= valid) sc[i] = neg_inf();
      }
      float mb = sc[0];
#pragma unroll
      for (int i = 1; i < IPB; ++i) mb = fmaxf(mb, sc[i]);
      const float mn = fmaxf(m[g], mb);
      if (mn == neg_inf()) continue;  // this row has seen no live token yet
      const float alpha = fast_exp2(m[g] - mn);  // 0 when m was -inf
      l[g] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
#pragma unroll
      for (int i = 0; i < IPB; ++i) {
        const float pi = fast_exp2(sc[i] - mn);  // 0 for masked tokens
        l[g] += pi;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(pi, vf[i][e], acc[g][e]);
      }
      m[g] = mn;
    }
  };

  // Two register sets alternate so the next block's loads are in flight
  // while the current one is computed. The steady-state loop issues its loads
  // unconditionally (a load under a branch makes the compiler wait for every
  // outstanding load at the join); the last one or two blocks are peeled.
  {
    Raw ka[IPB], va[IPB], kb[IPB], vb[IPB];
    const int last = nblk - 1;
    load(0, ka, va);
    int jb = 0;
    for (; jb + 2 < nblk; jb += 2) {
      load(jb + 1, kb, vb);
      compute(jb, ka, va);
      load(jb + 2, ka, va);
      compute(jb + 1, kb, vb);
    }
    if (jb + 1 < nblk) {
      load(min(jb + 1, last), kb, vb);
      compute(jb, ka, va);
      compute(jb + 1, kb, vb);
    } else {
      compute(jb, ka, va);
    }
  }

  // merge the row groups of the wave (lanes differing in the row bits)
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) {
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      const float mo = __shfl_xor(m[g], o, 64);
      const float lo = __shfl_xor(l[g], o, 64);
      const float M = fmaxf(m[g], mo);
      const float a1 = (m[g] == neg_inf()) ? 0.f : fast_exp2(m[g] - M);
      const float a2 = (mo == neg_inf()) ? 0.f : fast_exp2(mo - M);
      l[g] = l[g] * a1 + lo * a2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float ao = __shfl_xor(acc[g][e], o, 64);
        acc[g][e] = acc[g][e] * a1 + ao * a2;
      }
      m[g] = M;
    }
  }
  // lanes of row 0 hold the whole result: head g, dims c*EPL .. c*EPL+EPL-1
  if (r == 0) {
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
      if (g < p.G) {
        if constexpr (KV8) {  // the V scale multiplies the (partial) output
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[g][e] *= p.v_scale;
        }
        store_result<PRE>(p, w, nps, g, c * EPL, acc[g], EPL, m[g], l[g], c == 0, bad, D);
      }
  }
}

// ============================================================================
// Decode on MFMA matrix cores for grouped-query attention: f16/bf16, head_dim
// 128, 2..16 query heads sharing one KV head. Per 16-token block a wave forms
//   S^T[token][col] = K[token][:] . Q[col][:]       (4 x mfma 16x16x32)
//   O^T[d][col]   += V^T[d][token] . P^T[token][col]  (8 x mfma 16x16x16)
// The 16 MFMA columns are query heads. P stays in fp32 precision: each weight
// is split into a 16-bit high part and a 16-bit residual. With at most 8
// heads (SPLITCOL) the group's queries are placed twice, in columns 0..7 and
// 8..15; columns 0..7 carry the high parts and 8..15 the residuals through
// the same PV MFMA, and the two halves are added at the end. With 9..16 heads
// each tile takes two PV MFMAs, one per part.
//
// Register layouts (lane l, c = l % 16, g = l / 16):
//   16x16x32: A row c, k = 8g..8g+7;  B k = 8g..8g+7, column c;
//   16x16x16: A row c, k = 4g..4g+3;  B k = 4g..4g+3, column c;
//   C (both): rows 4g..4g+3, column c.
// K is loaded straight into the A layout of the score MFMA (lane: token c,
// dims 32kc+8g..+8). The score tile leaves lane l with column c, tokens
// 4g..4g+3 - exactly the lane's B operand of the PV product. V is loaded as
// whole 256-byte rows (lane: dims 8c..8c+7 of tokens 4g..4g+3) and regrouped
// with v_perm so that tile n holds dimension d = 8c + n in row c - no LDS
// transpose. The O^T accumulator then leaves lane l with column c, dims
// 32g..32g+31.
//
// The running max is updated lazily: a block's weights are taken against the
// current max unless some score exceeds it by more than kRescaleSlack
// (base-2 units), so most blocks skip the cross-lane max and the rescale of
// the accumulators; weights stay below 2^kRescaleSlack, far from overflow.
// ============================================================================
template <int DT, bool SPLITCOL, int RING, int BS, bool KV8, bool NT, bool PRE = false>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_mfma_kernel(DecodeParams p) {
  constexpr int D = 128;
  constexpr int kRowU4 = KV8 ? D / 16 : D / 8;  // uint4 per token row of the pools
  const int lane = threadIdx.x;
  const int u = blockIdx.x;
  if (u >= p.n_units) return;
  const int col = lane & 15;  // MFMA column / token row of a K tile
  const int grp = lane >> 4;  // k-slot group
  const WorkItem w = unit_item(p, u);
  if (!w.ok) return;
  // The loads that need only the unit go out together: the length, the
  // partition's table entries (bounded by the table width, so the length is
  // not needed yet) and the queries.
  const int ctx = p.lens[w.s] - p.skip_tokens;
  const int b0 = (p.skip_tokens + w.part * p.part_tokens) / BS;  // the partition's first entry
  Entries raw_entry{0, 0};
  {
    constexpr int K = entries_per_lane<BS>();
    const int32_t* row = p.tables + (size_t)w.s * p.max_blocks + b0;
    if (lane * K < p.max_blocks - b0) raw_entry.lo = row[lane * K];
    if (K == 2 && lane * K + 1 < p.max_blocks - b0) raw_entry.hi = row[lane * K + 1];
  }
  // B operand of the score MFMA: Q^T, lane holds head `hd`, dims 32kc+8grp..+8
  // (fp8 cache: dims 16grp+8kc.. for kc < 2 and 64+16grp+8(kc-2).. for kc >= 2,
  // the order in which a lane's two 16-byte K loads hold them)
  const int hd = SPLITCOL ? (col & 7) : col;
  const bool live_head = hd < p.G;
  uint4 qb[4];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(
        static_cast<const char*>(p.q) +
        (((size_t)w.s * p.Hq + (size_t)w.h * p.G + (live_head ? hd : 0)) * D) * 2);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const uint4 v = qp[KV8 ? (kc >> 1) * 8 + 2 * grp + (kc & 1) : kc * 4 + grp];
      qb[kc] = live_head ? v : make_uint4(0, 0, 0, 0);
    }
  }
  // With a fused cache write, the new token's K chunks kc*4+grp and V chunk
  // col are fetched in the same batch (whether or not this unit turns out to
  // hold the sequence's last position), so storing them costs no extra wait.
  uint4 kn0 = make_uint4(0, 0, 0, 0), kn1 = kn0, kn2 = kn0, kn3 = kn0, vnew = kn0;
  if (p.k_new) {
    const uint4* kn = static_cast<const uint4*>(p.k_new) + ((size_t)w.s * p.Hkv + w.h) * (D / 8);
    if constexpr (KV8) {  // the 16-bit chunks behind the lane's two fp8 K chunks
      kn0 = kn[2 * grp];
      kn1 = kn[2 * grp + 1];
      kn2 = kn[8 + 2 * grp];
      kn3 = kn[9 + 2 * grp];
    } else {
      kn0 = kn[grp];
      kn1 = kn[4 + grp];
      kn2 = kn[8 + grp];
      kn3 = kn[12 + grp];
    }
    vnew = (static_cast<const uint4*>(p.v_new) + ((size_t)w.s * p.Hkv + w.h) * (D / 8))[col];
  }
  const int nps = unit_prologue<D, PRE>(p, w, ctx, lane);
  if (nps == 0) return;
  const int t0 = w.part * p.part_tokens;
  const int t1 = min(ctx, t0 + p.part_tokens);
  const int nblk = (t1 - t0 + kTile - 1) / kTile;  // 16-token tiles
  const int last = nblk - 1;
  bool bad = false;
  const Entries staged = check_entries<BS>(p, raw_entry, (t1 - t0 + BS - 1) / BS, lane, bad);
  const NewToken nt = new_token<BS>(p, w, nps, ctx, t0, staged, bad, lane);
  if (nt.on && nt.slot >= 0) {
    // Each lane stores exactly the chunks of the new token's rows that it
    // later loads with the last block (K: the lanes of column nt.row, chunks
    // kc*4+grp; V: the lanes of row group nt.row/4, chunk col), so program
    // order within the lane makes that load return the new values.
    const size_t dst = tile_row<BS>(p, w.h, staged, last, nt.row, kRowU4);
    if constexpr (KV8) {
      // quantised: K chunks grp and 4+grp (16 codes each), V chunk col (8 codes)
      if (col == nt.row) {
        uint4* kd = static_cast<uint4*>(p.k_pool_w) + dst + grp;
        const uint2 a = e4m3x8_from16<DT>(kn0, p.k_scale), b = e4m3x8_from16<DT>(kn1, p.k_scale);
        const uint2 c = e4m3x8_from16<DT>(kn2, p.k_scale), d = e4m3x8_from16<DT>(kn3, p.k_scale);
        kd[0] = make_uint4(a.x, a.y, b.x, b.y);
        kd[4] = make_uint4(c.x, c.y, d.x, d.y);
      }
      if (grp == nt.row / 4)
        static_cast<uint2*>(p.v_pool_w)[2 * dst + col] = e4m3x8_from16<DT>(vnew, p.v_scale);
    } else {
      if (col == nt.row) {
        uint4* kd = static_cast<uint4*>(p.k_pool_w) + dst + grp;
        kd[0] = kn0;
        kd[4] = kn1;
        kd[8] = kn2;
        kd[12] = kn3;
      }
      if (grp == nt.row / 4) static_cast<uint4*>(p.v_pool_w)[dst + col] = vnew;
    }
  }

  const bool residual_lane = SPLITCOL && col >= 8;

  f32x4 o[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = neg_inf(), l = 0.f;

  const char* kbase = static_cast<const char*>(p.k_pool);
  const char* vbase = static_cast<const char*>(p.v_pool);

  // Raw tile data held per lane: 16-bit cache 4 K + 4 V uint4; fp8 cache
  // 2 K uint4 (16 codes each) + 4 V uint2 (8 codes each).
  constexpr int kKU = KV8 ? 2 : 4;
  typedef typename std::conditional<KV8, uint2, uint4>::type VRaw;
  auto load = [&](int j, uint4* ku, VRaw* vu) {
    // K: row col of the tile; V: rows 4grp..4grp+3 (consecutive in one block).
    // Rows past the tile's live tokens read the last live row (K) or row
    // group (V) instead - their values are masked - so the unused rows of a
    // sequence's last block are never fetched.
    const int lim = t1 - (t0 + j * kTile) - 1;  // last live row of tile j
    const int kr = min(col, lim), vg = min(grp, lim >> 2);
    const uint4* kt = reinterpret_cast<const uint4*>(kbase) + tile_row<BS>(p, w.h, staged, j, kr, kRowU4);
    if constexpr (KV8) {
      const uint2* vt = reinterpret_cast<const uint2*>(vbase) +
                        tile_row<BS>(p, w.h, staged, j, 4 * vg, 2 * kRowU4);
      ku[0] = load_kv<NT>(kt + grp);
      ku[1] = load_kv<NT>(kt + 4 + grp);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) vu[jj] = load_kv<NT>(vt + jj * 2 * kRowU4 + col);
    } else {
      const uint4* vt = reinterpret_cast<const uint4*>(vbase) +
                        tile_row<BS>(p, w.h, staged, j, 4 * vg, kRowU4);
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) ku[kc] = load_kv<NT>(kt + kc * 4 + grp);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) vu[jj] = load_kv<NT>(vt + jj * kRowU4 + col);
    }
  };

  auto compute16 = [&](int jb, uint4* ku, uint4* vu) {
    f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) st = mfma_qk<DT>(ku[kc], qb[kc], st);
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = st[r] * p.scale_log2;
    const int valid = t1 - (t0 + jb * kTile);  // live tokens of the tile (>= 1)
    if (valid < kTile) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * grp + r >= valid) {
          x[r] = neg_inf();
          vu[r] = make_uint4(0, 0, 0, 0);  // masked rows may hold NaN
        }
    }
    const float lm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    if (__builtin_amdgcn_ballot_w64(lm > m + kRescaleSlack) != 0) {
      const float mn = fmaxf(m, column_max(lm));
      const float alpha = fast_exp2(m - mn);  // 0 while m is -inf
      l *= alpha;
#pragma unroll
      for (int n = 0; n < 8; ++n) o[n] *= alpha;
      m = mn;
    }
    float pw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pw[r] = fast_exp2(x[r] - m);  // 0 for masked tokens
      l += pw[r];
    }
    if constexpr (SPLITCOL) {
      const uint2 ph = weight_part<DT>(pw, 0.0f);
      const uint2 pl = weight_part<DT>(pw, 1.0f);
      const uint2 pb = residual_lane ? pl : ph;
#pragma unroll
      for (int n = 0; n < 8; ++n) o[n] = mfma_pv<DT>(v_column(vu, n), pb, o[n]);
    } else {
      const uint2 ph = weight_part<DT>(pw, 0.0f);
      const uint2 pl = weight_part<DT>(pw, 1.0f);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const uint2 a = v_column(vu, n);
        o[n] = mfma_pv<DT>(a, ph, o[n]);
        o[n] = mfma_pv<DT>(a, pl, o[n]);
      }
    }
  };
  auto compute = [&](int jb, uint4* ku, VRaw* vu) {
    if constexpr (KV8) {
      // widen the codes to the query's 16-bit type (exact), then as above
      uint4 k16[4], v16[4];
      k16[0] = e4m3x8_widen<DT>(ku[0].x, ku[0].y);
      k16[1] = e4m3x8_widen<DT>(ku[0].z, ku[0].w);
      k16[2] = e4m3x8_widen<DT>(ku[1].x, ku[1].y);
      k16[3] = e4m3x8_widen<DT>(ku[1].z, ku[1].w);
#pragma unroll
      for (int r = 0; r < 4; ++r) v16[r] = e4m3x8_widen<DT>(vu[r].x, vu[r].y);
      compute16(jb, k16, v16);
    } else {
      compute16(jb, ku, vu);
    }
  };

  // Ring of RING blocks: while one block is computed the next RING-1 are in
  // flight. The prologue and the steady-state loop issue their loads
  // unconditionally (a load under a branch makes the compiler wait for every
  // outstanding load at the join); the last blocks are drained with guarded
  // refills.
  {
    uint4 kr[RING][kKU];
    VRaw vr[RING][4];
#pragma unroll
    for (int s = 0; s < RING; ++s) load(min(s, last), kr[s], vr[s]);
    int j = 0;
    for (; j + 2 * RING <= nblk; j += RING) {
#pragma unroll
      for (int s = 0; s < RING; ++s) {
        compute(j + s, kr[s], vr[s]);
        load(j + s + RING, kr[s], vr[s]);
      }
    }
#pragma unroll
    for (int s = 0; s < RING; ++s) {
      if (j + s < nblk) compute(j + s, kr[s], vr[s]);
      if (j + s + RING < nblk) load(j + s + RING, kr[s], vr[s]);
    }
#pragma unroll
    for (int s = 0; s < RING; ++s)
      if (j + RING + s < nblk) compute(j + RING + s, kr[s], vr[s]);
  }

  l = column_sum(l);
  if constexpr (SPLITCOL) {
    // column c < 8 adds the residual half held by column c + 8
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[n][r] += dpp<0x128>(o[n][r]);  // row_ror:8
  }
  // Stage the group's G x D results in LDS and write them back as contiguous
  // 1 KB spans: in the accumulator layout neighbouring lanes hold different
  // heads, 512 bytes apart in memory.
  __shared__ float stage[16 * kStageStride];
  __shared__ float stage_lse[16];  // shared-prefix step: log2 denominators per head
  const bool writer = SPLITCOL ? (col < 8 && live_head) : live_head;
  if (writer) {
    if constexpr (PRE)
      if (nps == 1 && grp == 0) stage_lse[hd] = m + log2f(l);
    // lane holds head hd, dims 32*grp + 8*r + n for r < 4, n < 8; an fp8
    // cache's V scale multiplies the (partial) output
    float inv = nps == 1 ? 1.0f / l : 1.0f;
    if constexpr (KV8) inv *= p.v_scale;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        *reinterpret_cast<float4*>(&stage[hd * kStageStride + 32 * grp + 8 * r + 4 * hh]) =
            make_float4(o[4 * hh][r] * inv, o[4 * hh + 1][r] * inv, o[4 * hh + 2][r] * inv,
                        o[4 * hh + 3][r] * inv);
  }
  __syncthreads();
  const size_t pg = partial_group(p, w);
  float* dst = nps == 1 ? p.out + ((size_t)w.s * p.Hq + (size_t)w.h * p.G) * D
                        : p.ws_o + pg * p.G * D;
  const float nan = __builtin_nanf("");
  const size_t row0 = (size_t)w.s * p.Hq + (size_t)w.h * p.G;
  for (int c = lane; c < p.G * (D / 4); c += 64) {
    float4 v = *reinterpret_cast<const float4*>(&stage[(c >> 5) * kStageStride + 4 * (c & 31)]);
    if (bad && nps == 1) v = make_float4(nan, nan, nan, nan);
    if constexpr (PRE)
      if (nps == 1)
        v = with_prefix(p, row0 + c / (D / 4), c % (D / 4), D / 4, v,
                        bad ? nan : stage_lse[c / (D / 4)]);
    *reinterpret_cast<float4*>(dst + (size_t)c * 4) = v;
  }
  if (nps > 1 && writer && grp == 0)
    *reinterpret_cast<float2*>(p.ws_ml + (pg * p.G + hd) * 2) =
        bad ? make_float2(nan, nan) : make_float2(m, l);
}

inline int32_t effective_partition(int32_t partition_size) {
  return partition_size == 0 ? kDefaultPartition : partition_size;
}

// One wave64 workgroup per work unit.
template <typename Kernel>
kv_status launch_decode(Kernel kernel, const DecodeParams& prm, hipStream_t st) {
  hipLaunchKernelGGL(kernel, dim3((unsigned)prm.n_units), dim3(64), 0, st, prm);
  return launch_status("kv_paged_attention_decode");
}

template <int DT, int D, int BS, bool NT, bool KV8 = false>
kv_status launch_valu(const DecodeParams& prm, int gmax, hipStream_t st) {
  switch (gmax) {
    case 1: return launch_decode(decode_valu_kernel<DT, D, 1, BS, NT, false, KV8>, prm, st);
    case 2: return launch_decode(decode_valu_kernel<DT, D, 2, BS, NT, false, KV8>, prm, st);
    case 4: return launch_decode(decode_valu_kernel<DT, D, 4, BS, NT, false, KV8>, prm, st);
    case 8: return launch_decode(decode_valu_kernel<DT, D, 8, BS, NT, false, KV8>, prm, st);
    case 16: return launch_decode(decode_valu_kernel<DT, D, 16, BS, NT, false, KV8>, prm, st);
    default: return fail(KV_ERR_UNSUPPORTED, "decode: group size");
  }
}

inline int group_bucket(int G) { return G == 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : G <= 8 ? 8 : 16; }

// The decode kernel for one block size: MFMA for grouped 16-bit heads of
// dimension 128, vector ALUs otherwise.
template <int BS, bool NT>
kv_status launch_decode_kernel(const DecodeParams& prm, kv_dtype dtype, int head_dim, int G,
                               hipStream_t st) {
  constexpr int R = kDecodeRing;
  if (prm.pre_parts) {
    // the shared-prefix step's tails (16-bit, head_dim 128): the variants that
    // fold the prefix ranges into the outputs
    if (G == 1)
      return dtype == KV_BF16
                 ? launch_decode(decode_valu_kernel<KV_BF16, 128, 1, BS, NT, true>, prm, st)
                 : launch_decode(decode_valu_kernel<KV_F16, 128, 1, BS, NT, true>, prm, st);
    constexpr int RP = kDecodeRingPre;
    if (G <= 8)
      return dtype == KV_BF16
                 ? launch_decode(decode_mfma_kernel<KV_BF16, true, RP, BS, false, NT, true>, prm, st)
                 : launch_decode(decode_mfma_kernel<KV_F16, true, RP, BS, false, NT, true>, prm, st);
    return dtype == KV_BF16
               ? launch_decode(decode_mfma_kernel<KV_BF16, false, RP, BS, false, NT, true>, prm, st)
               : launch_decode(decode_mfma_kernel<KV_F16, false, RP, BS, false, NT, true>, prm, st);
  }
  if ((dtype == KV_F16 || dtype == KV_BF16) && head_dim == 128 && G >= 2) {
    if (G <= 8)
      return dtype == KV_BF16
                 ? launch_decode(decode_mfma_kernel<KV_BF16, true, R, BS, false, NT>, prm, st)
                 : launch_decode(decode_mfma_kernel<KV_F16, true, R, BS, false, NT>, prm, st);
    return dtype == KV_BF16
               ? launch_decode(decode_mfma_kernel<KV_BF16, false, R, BS, false, NT>, prm, st)
               : launch_decode(decode_mfma_kernel<KV_F16, false, R, BS, false, NT>, prm, st);
  }
  const int gmax = group_bucket(G);
  if (dtype == KV_F32)
    return head_dim == 64 ? launch_valu<KV_F32, 64, BS, NT>(prm, gmax, st)
                          : launch_valu<KV_F32, 128, BS, NT>(prm, gmax, st);
  if (dtype == KV_F16)  // 16-bit head_dim 128 reaches here only with G == 1
    return head_dim == 64 ? launch_valu<KV_F16, 64, BS, NT>(prm, gmax, st)
                          : launch_decode(decode_valu_kernel<KV_F16, 128, 1, BS, NT>, prm, st);
  return head_dim == 64 ? launch_valu<KV_BF16, 64, BS, NT>(prm, gmax, st)
                        : launch_decode(decode_valu_kernel<KV_BF16, 128, 1, BS, NT>, prm, st);
}

// fp8 cache, f16 or bf16 queries: the MFMA kernel for every group size
// (1..16) at head_dim 128, the vector-ALU kernel at head_dim 64; the
// shared-prefix step's tails (head_dim 128) take the MFMA variants that fold
// the prefix ranges into the outputs.
template <int BS, bool NT>
kv_status launch_decode_kernel_fp8(const DecodeParams& prm, kv_dtype dtype, int head_dim, int G,
                                   hipStream_t st) {
  constexpr int R = kDecodeRing8;
  if (prm.pre_parts) {
    if (G <= 8)
      return dtype == KV_BF16
                 ? launch_decode(decode_mfma_kernel<KV_BF16, true, R, BS, true, NT, true>, prm, st)
                 : launch_decode(decode_mfma_kernel<KV_F16, true, R, BS, true, NT, true>, prm, st);
    return dtype == KV_BF16
               ? launch_decode(decode_mfma_kernel<KV_BF16, false, R, BS, true, NT, true>, prm, st)
               : launch_decode(decode_mfma_kernel<KV_F16, false, R, BS, true, NT, true>, prm, st);
  }
  if (head_dim == 64)
    return dtype == KV_BF16 ? launch_valu<KV_BF16, 64, BS, NT, true>(prm, group_bucket(G), st)
                            : launch_valu<KV_F16, 64, BS, NT, true>(prm, group_bucket(G), st);
  if (G <= 8)
    return dtype == KV_BF16
               ? launch_decode(decode_mfma_kernel<KV_BF16, true, R, BS, true, NT>, prm, st)
               : launch_decode(decode_mfma_kernel<KV_F16, true, R, BS, true, NT>, prm, st);
  return dtype == KV_BF16
             ? launch_decode(decode_mfma_kernel<KV_BF16, false, R, BS, true, NT>, prm, st)
             : launch_decode(decode_mfma_kernel<KV_F16, false, R, BS, true, NT>, prm, st);
}

// The launchers of one (block size, load policy), instantiated in
// decode_variants.hip.
#define PAGEDKV_DECODE_LAUNCHERS(EXTERN, BS, NT)                                         \
  EXTERN template kv_status launch_decode_kernel<BS, NT>(const DecodeParams&, kv_dtype, int, \
                                                         int, hipStream_t);              \
  EXTERN template kv_status launch_decode_kernel_fp8<BS, NT>(const DecodeParams&, kv_dtype, \
                                                             int, int, hipStream_t);

}  // namespace decode
}  // namespace pagedkv

#endif  // PAGEDKV_DECODE_KERNELS_H_
