// Device side of pagedkv for AMD CDNA4 (gfx950): slot mapping, cache scatter,
// copy-on-write block copy, paged decode attention and the split-K merge.
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
// Work split: one workgroup (4 wave64s) per (sequence, KV head, context
// partition). The partition's block-table entries are staged in LDS first, so
// every K/V address is known before the first load. Each wave walks every
// fourth 16-token block of the partition, keeps an online softmax (running
// max and sum, [2] "The Custom CUDA Kernel"), and the four waves merge in
// LDS. Sequences longer than one partition write unnormalised partial results
// that a second kernel merges with the log-sum-exp rule.
//
// Softmax runs in base 2: scores are multiplied by scale*log2(e) and
// exponentiated with v_exp_f32; the result is the same softmax.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/pagedkv.h"
#include "status.h"

using pagedkv::fail;

namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;

constexpr int kBlock = 16;          // tokens per KV block (device kernels)
constexpr int kWaves = 4;           // wave64s per decode workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxPartition = 8192; // tokens
constexpr int kDefaultPartition = 512;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- element conversion -----------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffffu));
}
__device__ __forceinline__ float f16hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}

// Unpack one 16-byte chunk into fp32 values (4 for fp32, 8 for 16-bit types).
template <int DT>
__device__ __forceinline__ void unpack16(const uint4& u, float* f) {
  if constexpr (DT == KV_F32) {
    f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
  } else if constexpr (DT == KV_BF16) {
    f[0] = bf16lo(u.x); f[1] = bf16hi(u.x); f[2] = bf16lo(u.y); f[3] = bf16hi(u.y);
    f[4] = bf16lo(u.z); f[5] = bf16hi(u.z); f[6] = bf16lo(u.w); f[7] = bf16hi(u.w);
  } else {
    f[0] = f16lo(u.x); f[1] = f16hi(u.x); f[2] = f16lo(u.y); f[3] = f16hi(u.y);
    f[4] = f16lo(u.z); f[5] = f16hi(u.z); f[6] = f16lo(u.w); f[7] = f16hi(u.w);
  }
}

// ---- cross-lane reductions --------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over groups of LPR consecutive lanes (LPR = 8, 16 or 32). Within a
// 16-lane DPP row: swap neighbours, swap pairs, mirror halves, mirror the row.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (LPR >= 16) x += dpp<0x140>(x);  // row_mirror
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16, 64);
  return x;
}

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

// ---- shared decode parameters ----------------------------------------------
struct DecodeParams {
  float* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* tables;
  const int32_t* lens;
  const int32_t* items;  // optional work plan: [n_items][2] = (sequence, partition)
  float* ws_o;           // [S][Hq][nparts][D]   partial outputs (unnormalised)
  float* ws_ml;          // [S][Hq][nparts][2]   partial (max, sum) in base-2 units
  int32_t max_blocks, S, Hq, Hkv, G, num_blocks, part_tokens, nparts, n_units;
  float scale_log2;
};

// Every wave64 is an independent worker: wave `u` of the grid processes work
// unit u, one (sequence, KV head, context partition), from its first block
// to its last, and writes its result itself - the normalised output when the
// sequence has a single partition, else an unnormalised partial result for
// the split-K merge. There is no cross-wave merge, no LDS and no barrier, so
// nothing stalls one wave on another. With a plan, u = item * Hkv + head and
// the items are sorted longest first: the four waves of a workgroup get
// units of similar size and finish together, and the hardware dispatcher
// balances the tail. Without a plan, u enumerates (partition, head,
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

// Sequence-level checks shared by both decode kernels (one wave). Returns the
// number of partitions of the sequence when this unit has tokens to process,
// else 0 (the output of an empty or invalid sequence is written by its
// partition-0 unit: zeros, or NaN for a length that is negative or exceeds
// the table or max_context_len).
template <int D>
__device__ __forceinline__ int unit_prologue(const DecodeParams& p, const WorkItem& w, int ctx,
                                             int lane) {
  const bool bad = ctx < 0 || (int64_t)ctx > (int64_t)p.max_blocks * kBlock ||
                   (int64_t)ctx > (int64_t)p.nparts * p.part_tokens;
  if (bad || ctx == 0) {
    if (w.part == 0) {
      const float v = bad ? __builtin_nanf("") : 0.0f;
      float* dst = p.out + ((size_t)w.s * p.Hq + (size_t)w.h * p.G) * D;
      for (int i = lane; i < p.G * D; i += 64) dst[i] = v;
    }
    return 0;
  }
  const int nps = (ctx + p.part_tokens - 1) / p.part_tokens;
  return w.part < nps ? nps : 0;
}

// Physical block of logical block `jb` of the unit's partition, read through
// the scalar cache (the index is wave-uniform). An ID outside the pool marks
// the unit invalid and is read as block 0, so no load leaves the pool.
__device__ __forceinline__ int block_id(const DecodeParams& p, const int32_t* row, int jb,
                                        bool& bad) {
  int e = row[jb];
  if (e < 0 || e >= p.num_blocks) {
    bad = true;
    e = 0;
  }
  return e;
}

// Store `n` consecutive floats of head `hq` starting at dimension d0: the
// final output o / l for a single-partition sequence, else the partial
// result o (and, from the lane with `write_ml`, the pair (m, l)). An invalid
// unit stores NaN.
__device__ __forceinline__ void store_result(const DecodeParams& p, const WorkItem& w, int nps,
                                             int hq, int d0, const float* o, int n, float m,
                                             float l, bool write_ml, bool bad, int D) {
  const float nan = __builtin_nanf("");
  if (nps == 1) {
    float* dst = p.out + ((size_t)w.s * p.Hq + hq) * D + d0;
    const float inv = 1.0f / l;
    for (int i = 0; i < n; i += 4) {
      float4 v = make_float4(o[i] * inv, o[i + 1] * inv, o[i + 2] * inv, o[i + 3] * inv);
      if (bad) v = make_float4(nan, nan, nan, nan);
      *reinterpret_cast<float4*>(dst + i) = v;
    }
  } else {
    const size_t slot = ((size_t)w.s * p.Hq + hq) * p.nparts + w.part;
    float* dst = p.ws_o + slot * D + d0;
    for (int i = 0; i < n; i += 4)
      *reinterpret_cast<float4*>(dst + i) = make_float4(o[i], o[i + 1], o[i + 2], o[i + 3]);
    if (write_ml)
      *reinterpret_cast<float2*>(p.ws_ml + slot * 2) = bad ? make_float2(nan, nan)
                                                            : make_float2(m, l);
  }
}

// ============================================================================
// Decode on the vector ALUs: any dtype, head_dim 64/128, up to GMAX query
// heads per KV head. Each token row of a block is spread over LPR lanes
// (16 bytes per lane), so one dwordx4 load per lane reads TPI whole rows and a
// 16-token block takes IPB loads. Dot products are finished with DPP row
// reductions. Each group of LPR lanes keeps its own online softmax over the
// tokens it reads; the groups are merged with cross-lane shuffles at the end.
// ============================================================================
template <int DT, int D, int GMAX>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(DecodeParams p) {
  constexpr int EB = DT == KV_F32 ? 4 : 2;
  constexpr int EPL = 16 / EB;           // elements per lane chunk
  constexpr int LPR = D * EB / 16;       // lanes per token row
  constexpr int TPI = 64 / LPR;          // rows per wave-wide load
  constexpr int IPB = kBlock / TPI;      // loads per 16-token block
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "unsupported row width");

  const int lane = threadIdx.x & 63;
  const int u = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (u >= p.n_units) return;
  const int r = lane / LPR, c = lane % LPR;
  const WorkItem w = unit_item(p, u);
  if (!w.ok) return;
  const int ctx = p.lens[w.s];
  const int nps = unit_prologue<D>(p, w, ctx, lane);
  if (nps == 0) return;
  const int t0 = w.part * p.part_tokens;
  const int t1 = min(ctx, t0 + p.part_tokens);
  const int nblk = (t1 - t0 + kBlock - 1) / kBlock;
  const int32_t* row = p.tables + (size_t)w.s * p.max_blocks + t0 / kBlock;
  bool bad = false;

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

  const size_t tile_u4 = (size_t)kBlock * LPR;  // uint4 per (block, head) tile
  const uint4* kbase = static_cast<const uint4*>(p.k_pool);
  const uint4* vbase = static_cast<const uint4*>(p.v_pool);

  auto load = [&](int e, uint4* ku, uint4* vu) {
    const size_t tile = ((size_t)e * p.Hkv + w.h) * tile_u4;
#pragma unroll
    for (int i = 0; i < IPB; ++i) ku[i] = kbase[tile + (size_t)(r + TPI * i) * LPR + c];
#pragma unroll
    for (int i = 0; i < IPB; ++i) vu[i] = vbase[tile + (size_t)(r + TPI * i) * LPR + c];
  };

  auto compute = [&](int jb, const uint4* ku, const uint4* vu) {
    const int valid = t1 - (t0 + jb * kBlock);  // live tokens in this block (>= 1)
    const bool full = valid >= kBlock;
    float kf[IPB][EPL], vf[IPB][EPL];
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      unpack16<DT>(ku[i], kf[i]);
      unpack16<DT>(vu[i], vf[i]);
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
  // unconditionally (a load under a branch would force a wait for every
  // outstanding load at the join); the last one or two blocks are peeled.
  {
    uint4 ka[IPB], va[IPB], kb[IPB], vb[IPB];
    const int last = nblk - 1;
    int eb = block_id(p, row, min(1, last), bad);
    load(block_id(p, row, 0, bad), ka, va);
    int jb = 0;
    for (; jb + 2 < nblk; jb += 2) {
      const int ea2 = block_id(p, row, jb + 2, bad);
      load(eb, kb, vb);
      compute(jb, ka, va);
      eb = block_id(p, row, min(jb + 3, last), bad);
      load(ea2, ka, va);
      compute(jb + 1, kb, vb);
    }
    if (jb + 1 < nblk) {
      load(eb, kb, vb);
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
      if (g < p.G)
        store_result(p, w, nps, w.h * p.G + g, c * EPL, acc[g], EPL, m[g], l[g], c == 0, bad, D);
  }
}

// ============================================================================
// Decode on MFMA matrix cores for grouped-query attention: f16/bf16, head_dim
// 128, 2..16 query heads sharing one KV head. Per 16-token block a wave forms
//   S^T[token][head] = K[token][:] . Q[head][:]   (4 x mfma 16x16x32)
//   O^T[d][head]   += V^T[d][token] . P^T[token][head]   (16 x mfma 16x16x16)
// The group's heads are the 16 MFMA columns (unused columns are zero). K is
// loaded straight into the A-operand layout (lane l: token l%16, 8 dims at
// 32*kc + 8*(l/16)); V is loaded as whole 256-byte rows (lane l: dims
// 8*(l%16)..+8 of token 4*(l/16)+jj) and regrouped in registers so that lane l
// feeds d = 8*(l%16)+n of tile n - no LDS transpose. The S^T output layout
// (lane l: head l%16, tokens 4*(l/16)+r) is exactly the B operand P^T needs,
// and the O^T accumulator leaves lane l with head l%16, dims 32*(l/16)..+32.
// P stays in fp32 precision: it is split into a 16-bit high part and a 16-bit
// residual and both go through the PV MFMA, so the products are accumulated
// in fp32 with no 16-bit rounding of the weights.
// ============================================================================
template <int DT>
__device__ __forceinline__ f32x4 mfma_qk(const uint4& a, const uint4& b, f32x4 c) {
  if constexpr (DT == KV_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ f32x4 mfma_pv(const uint2& a, const uint2& b, f32x4 c) {
  if constexpr (DT == KV_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// Split an fp32 weight into a 16-bit high part and a 16-bit residual.
template <int DT>
__device__ __forceinline__ void split_weight(float x, uint32_t& hi, uint32_t& lo) {
  if constexpr (DT == KV_BF16) {
    const uint32_t xb = __float_as_uint(x);
    hi = xb >> 16;  // truncation; the residual below is exact in fp32
    const float rem = x - __uint_as_float(xb & 0xffff0000u);
    const uint32_t rb = __float_as_uint(rem);
    lo = (rb + 0x7fffu + ((rb >> 16) & 1u)) >> 16;  // round to nearest even
  } else {
    const _Float16 h = (_Float16)x;
    const _Float16 r = (_Float16)(x - (float)h);
    hi = __builtin_bit_cast(unsigned short, h);
    lo = __builtin_bit_cast(unsigned short, r);
  }
}

// 16-bit element n (0..7) of four 16-byte chunks, packed as the MFMA operand
// (element of chunk 0 in the low half of the first dword).
__device__ __forceinline__ uint2 gather_col(const uint4* v, int n) {
  auto word = [](const uint4& u, int k) -> uint32_t {
    return k == 0 ? u.x : (k == 1 ? u.y : (k == 2 ? u.z : u.w));
  };
  const uint32_t w0 = word(v[0], n >> 1), w1 = word(v[1], n >> 1);
  const uint32_t w2 = word(v[2], n >> 1), w3 = word(v[3], n >> 1);
  uint2 r;
  if (n & 1) {
    r.x = (w0 >> 16) | (w1 & 0xffff0000u);
    r.y = (w2 >> 16) | (w3 & 0xffff0000u);
  } else {
    r.x = (w0 & 0xffffu) | (w1 << 16);
    r.y = (w2 & 0xffffu) | (w3 << 16);
  }
  return r;
}

template <int DT>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(DecodeParams p) {
  constexpr int D = 128;
  constexpr size_t kTileBytes = (size_t)kBlock * D * 2;  // 4 KB
  const int lane = threadIdx.x & 63;
  const int u = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (u >= p.n_units) return;
  const int col = lane & 15;  // MFMA column: query head of the group / token row
  const int grp = lane >> 4;  // k-slot group
  const WorkItem w = unit_item(p, u);
  if (!w.ok) return;
  const int ctx = p.lens[w.s];
  const int nps = unit_prologue<D>(p, w, ctx, lane);
  if (nps == 0) return;
  const int t0 = w.part * p.part_tokens;
  const int t1 = min(ctx, t0 + p.part_tokens);
  const int nblk = (t1 - t0 + kBlock - 1) / kBlock;
  const int32_t* row = p.tables + (size_t)w.s * p.max_blocks + t0 / kBlock;
  bool bad = false;

  // B operand of the score MFMA: Q^T, lane holds head `col`, dims 32kc+8grp..+8
  uint4 qb[4];
  {
    const bool live = col < p.G;
    const uint4* qp = reinterpret_cast<const uint4*>(
        static_cast<const char*>(p.q) +
        (((size_t)w.s * p.Hq + (size_t)w.h * p.G + (live ? col : 0)) * D) * 2);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const uint4 v = qp[kc * 4 + grp];
      qb[kc] = live ? v : make_uint4(0, 0, 0, 0);
    }
  }

  f32x4 o[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = neg_inf(), l = 0.f;

  const char* kbase = static_cast<const char*>(p.k_pool);
  const char* vbase = static_cast<const char*>(p.v_pool);

  auto load = [&](int e, uint4* ku, uint4* vu) {
    const size_t tile = ((size_t)e * p.Hkv + w.h) * kTileBytes;
    const uint4* kt = reinterpret_cast<const uint4*>(kbase + tile);
    const uint4* vt = reinterpret_cast<const uint4*>(vbase + tile);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) ku[kc] = kt[col * 16 + kc * 4 + grp];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) vu[jj] = vt[(4 * grp + jj) * 16 + col];
  };

  auto compute = [&](int jb, const uint4* ku, uint4* vu) {
    f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) st = mfma_qk<DT>(ku[kc], qb[kc], st);

    const int valid = t1 - (t0 + jb * kBlock);
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = st[r] * p.scale_log2;
    if (valid < kBlock) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * grp + r >= valid) {
          sc[r] = neg_inf();
          vu[r] = make_uint4(0, 0, 0, 0);  // masked rows may hold NaN
        }
    }
    float mb = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    const float mn = fmaxf(m, mb);  // finite: every block has a live token
    const float alpha = fast_exp2(m - mn);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int n = 0; n < 8; ++n) o[n] *= alpha;

    uint32_t hi[4], lo[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pr = fast_exp2(sc[r] - mn);
      l += pr;
      split_weight<DT>(pr, hi[r], lo[r]);
    }
    const uint2 phi = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
    const uint2 plo = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const uint2 a = gather_col(vu, n);
      o[n] = mfma_pv<DT>(a, phi, o[n]);
      o[n] = mfma_pv<DT>(a, plo, o[n]);
    }
  };

  // Two register sets alternate so the next block's loads are in flight
  // while the current block is computed. The steady-state loop issues its
  // loads unconditionally (a load under a branch would force a wait for every
  // outstanding load at the join); the last one or two blocks are peeled.
  {
    uint4 ka[4], va[4], kb[4], vb[4];
    const int last = nblk - 1;
    int eb = block_id(p, row, min(1, last), bad);
    load(block_id(p, row, 0, bad), ka, va);
    int jb = 0;
    for (; jb + 2 < nblk; jb += 2) {
      const int ea2 = block_id(p, row, jb + 2, bad);
      load(eb, kb, vb);
      compute(jb, ka, va);
      eb = block_id(p, row, min(jb + 3, last), bad);
      load(ea2, ka, va);
      compute(jb + 1, kb, vb);
    }
    if (jb + 1 < nblk) {
      load(eb, kb, vb);
      compute(jb, ka, va);
      compute(jb + 1, kb, vb);
    } else {
      compute(jb, ka, va);
    }
  }

  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (col < p.G) {
    // lane holds head `col`, dims 32*grp + 8*r + n for r < 4, n < 8
    float res[32];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int n = 0; n < 8; ++n) res[8 * r + n] = o[n][r];
    store_result(p, w, nps, w.h * p.G + col, 32 * grp, res, 32, m, l, grp == 0, bad, D);
  }
}

// ============================================================================
// Split-K merge ([2], "The Custom CUDA Kernel": partial outputs and softmax
// denominators computed per piece, then merged with a numerically stable
// rule). One workgroup per (sequence, query head) whose sequence has more
// than one partition; thread d merges dimension d in partition order:
//   M = max_k m_k,  L = sum_k l_k 2^(m_k - M),  out = sum_k 2^(m_k - M) o_k / L.
// A NaN denominator (invalid table entry) makes the output NaN. All partial
// (max, sum) pairs of the sequence are read by independent loads before use.
// ============================================================================
template <int D>
__global__ __launch_bounds__(D) void splitk_merge_kernel(float* __restrict__ out,
                                                         const float* __restrict__ ws_o,
                                                         const float* __restrict__ ws_ml,
                                                         const int32_t* __restrict__ lens,
                                                         int32_t Hq, int32_t nparts,
                                                         int32_t part_tokens,
                                                         int32_t max_blocks) {
  const int hq = blockIdx.x, s = blockIdx.y, d = threadIdx.x;
  const int ctx = lens[s];
  if (ctx <= 0 || (int64_t)ctx > (int64_t)max_blocks * kBlock ||
      (int64_t)ctx > (int64_t)nparts * part_tokens)
    return;  // written by the decode kernel
  const int nps = (ctx + part_tokens - 1) / part_tokens;
  if (nps <= 1) return;
  const size_t base = ((size_t)s * Hq + hq) * nparts;
  const float2* ml = reinterpret_cast<const float2*>(ws_ml) + base;
  float M = neg_inf();
  bool bad = false;
  for (int k = 0; k < nps; ++k) {
    const float2 v = ml[k];
    bad |= (v.y != v.y);
    M = fmaxf(M, v.x);
  }
  float L = 0.f, O = 0.f;
  for (int k = 0; k < nps; ++k) {
    const float2 v = ml[k];
    const float f = fast_exp2(v.x - M);
    L += v.y * f;
    O += ws_o[(base + k) * D + d] * f;
  }
  out[((size_t)s * Hq + hq) * D + d] = bad ? __builtin_nanf("") : O / L;
}

// ============================================================================
// Slot mapping ([4], "How it works"): slot = table[p / B] * B + p % B.
// ============================================================================
__global__ void slot_mapping_kernel(const int32_t* __restrict__ tables, int32_t num_rows,
                                    int32_t max_blocks, const int32_t* __restrict__ seq_idx,
                                    const int32_t* __restrict__ pos, int32_t n, int32_t B,
                                    int64_t* __restrict__ slots) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t s = seq_idx[i], p = pos[i];
  int64_t out = -1;
  if (s >= 0 && s < num_rows && p >= 0 && p / B < max_blocks) {
    const int32_t e = tables[(size_t)s * max_blocks + p / B];
    if (e >= 0) out = (int64_t)e * B + p % B;
  }
  slots[i] = out;
}

// ============================================================================
// reshape_and_cache ([3], "The allocation lifecycle"): copy each new token's
// K and V rows (all KV heads) into its slot. One thread moves 16 bytes of K
// and 16 bytes of V; consecutive threads cover consecutive bytes of a token,
// so reads and writes are coalesced per head row.
// ============================================================================
__global__ void reshape_and_cache_kernel(const uint4* __restrict__ k_new,
                                         const uint4* __restrict__ v_new,
                                         uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
                                         const int64_t* __restrict__ slots, int32_t n,
                                         int64_t num_slots, int32_t Hkv, int32_t row_u4,
                                         int32_t B) {
  const int64_t per_token = (int64_t)Hkv * row_u4;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)n * per_token) return;
  const int64_t i = t / per_token;
  const int64_t c = t % per_token;
  const int64_t h = c / row_u4, cc = c % row_u4;
  const int64_t slot = slots[i];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / B, off = slot % B;
  const int64_t dst = ((blk * Hkv + h) * B + off) * row_u4 + cc;
  k_pool[dst] = k_new[t];
  v_pool[dst] = v_new[t];
}

// ============================================================================
// Block copy for copy-on-write ([2], "Copy-on-Write ..."): blockIdx.x = pair,
// blockIdx.y = layer within this launch's chunk, blockIdx.z = 0 (K) / 1 (V).
// ============================================================================
constexpr int kCopyLayers = 64;
struct CopyPools {
  uint4* k[kCopyLayers];
  uint4* v[kCopyLayers];
};

__global__ void copy_blocks_kernel(CopyPools pools, const int32_t* __restrict__ pairs,
                                   int32_t num_blocks, int64_t block_u4) {
  const int32_t src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint4* base = blockIdx.z == 0 ? pools.k[blockIdx.y] : pools.v[blockIdx.y];
  const uint4* s = base + (int64_t)src * block_u4;
  uint4* d = base + (int64_t)dst * block_u4;
  for (int64_t i = threadIdx.x; i < block_u4; i += blockDim.x) d[i] = s[i];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

kv_status launch_status(const char* who) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KV_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return KV_OK;
}

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

int32_t effective_partition(int32_t partition_size) {
  return partition_size == 0 ? kDefaultPartition : partition_size;
}

// One wave per work unit, four waves per workgroup.
template <typename Kernel>
kv_status launch_decode(Kernel kernel, const DecodeParams& prm, hipStream_t st) {
  const int64_t grid = ((int64_t)prm.n_units + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, st, prm);
  return launch_status("kv_paged_attention_decode");
}

template <int DT, int D>
kv_status launch_valu(const DecodeParams& prm, int gmax, hipStream_t st) {
  switch (gmax) {
    case 1: return launch_decode(decode_valu_kernel<DT, D, 1>, prm, st);
    case 2: return launch_decode(decode_valu_kernel<DT, D, 2>, prm, st);
    case 4: return launch_decode(decode_valu_kernel<DT, D, 4>, prm, st);
    case 8: return launch_decode(decode_valu_kernel<DT, D, 8>, prm, st);
    case 16: return launch_decode(decode_valu_kernel<DT, D, 16>, prm, st);
    default: return fail(KV_ERR_UNSUPPORTED, "decode: group size");
  }
}

}  // namespace

extern "C" {

kv_status kv_slot_mapping(const int32_t* tables, int32_t num_rows, int32_t max_blocks,
                          const int32_t* seq_idx, const int32_t* pos, int32_t n,
                          int32_t block_size, int64_t* slots, hipStream_t stream) {
  pagedkv::clear_error();
  if (n < 0 || num_rows < 0 || max_blocks < 0 || block_size <= 0)
    return fail(KV_ERR_INVALID, "kv_slot_mapping: negative or zero size");
  if (n == 0) return KV_OK;
  if (!tables || !seq_idx || !pos || !slots)
    return fail(KV_ERR_INVALID, "kv_slot_mapping: null pointer");
  hipLaunchKernelGGL(slot_mapping_kernel, dim3((unsigned)ceil_div64(n, 256)), dim3(256), 0,
                     stream, tables, num_rows, max_blocks, seq_idx, pos, n, block_size, slots);
  return launch_status("kv_slot_mapping");
}

kv_status kv_reshape_and_cache(const void* k_new, const void* v_new, void* k_pool,
                               void* v_pool, const int64_t* slots, int32_t n,
                               int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, kv_dtype dtype, hipStream_t stream) {
  pagedkv::clear_error();
  const size_t eb = pagedkv::dtype_bytes(dtype);
  if (eb == 0) return fail(KV_ERR_UNSUPPORTED, "kv_reshape_and_cache: unknown dtype");
  if (n < 0 || num_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
    return fail(KV_ERR_INVALID, "kv_reshape_and_cache: bad sizes");
  if ((head_dim * eb) % 16 != 0)
    return fail(KV_ERR_UNSUPPORTED, "kv_reshape_and_cache: head_dim*elem must be a multiple of 16 bytes");
  if (n == 0) return KV_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !slots)
    return fail(KV_ERR_INVALID, "kv_reshape_and_cache: null pointer");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(KV_ERR_INVALID, "kv_reshape_and_cache: pointers must be 16-byte aligned");
  const int32_t row_u4 = (int32_t)(head_dim * eb / 16);
  const int64_t total = (int64_t)n * num_kv_heads * row_u4;
  const int64_t blocks = ceil_div64(total, 256);
  if (blocks > INT32_MAX) return fail(KV_ERR_INVALID, "kv_reshape_and_cache: too many tokens");
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                     static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool), slots, n,
                     (int64_t)num_blocks * block_size, num_kv_heads, row_u4, block_size);
  return launch_status("kv_reshape_and_cache");
}

kv_status kv_copy_blocks(void* const* k_pools, void* const* v_pools, int32_t num_layers,
                         const int32_t* pairs, int32_t n, int32_t num_blocks,
                         size_t block_bytes, hipStream_t stream) {
  pagedkv::clear_error();
  if (n < 0 || num_layers < 0 || num_layers > 256 || num_blocks <= 0)
    return fail(KV_ERR_INVALID, "kv_copy_blocks: bad sizes");
  if (block_bytes == 0 || block_bytes % 16 != 0)
    return fail(KV_ERR_INVALID, "kv_copy_blocks: block_bytes must be a positive multiple of 16");
  if (n == 0 || num_layers == 0) return KV_OK;
  if (!k_pools || !v_pools || !pairs) return fail(KV_ERR_INVALID, "kv_copy_blocks: null pointer");
  for (int32_t i = 0; i < num_layers; ++i)
    if (!k_pools[i] || !v_pools[i] || !aligned16(k_pools[i]) || !aligned16(v_pools[i]))
      return fail(KV_ERR_INVALID, "kv_copy_blocks: layer %d pool null or misaligned", i);
  for (int32_t l0 = 0; l0 < num_layers; l0 += kCopyLayers) {
    CopyPools cp{};
    const int32_t nl = num_layers - l0 < kCopyLayers ? num_layers - l0 : kCopyLayers;
    for (int32_t i = 0; i < nl; ++i) {
      cp.k[i] = static_cast<uint4*>(k_pools[l0 + i]);
      cp.v[i] = static_cast<uint4*>(v_pools[l0 + i]);
    }
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(n, nl, 2), dim3(256), 0, stream, cp, pairs,
                       num_blocks, (int64_t)(block_bytes / 16));
    kv_status st = launch_status("kv_copy_blocks");
    if (st != KV_OK) return st;
  }
  return KV_OK;
}

size_t kv_paged_attention_workspace_bytes(int32_t S, int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t max_context_len,
                                          int32_t partition_size) {
  const int32_t P = effective_partition(partition_size);
  if (S < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_context_len < 0 ||
      P <= 0)
    return 0;
  const int64_t nparts = ceil_div64(max_context_len, P);
  if (nparts <= 1) return 0;
  // partial outputs, then (max, sum) pairs
  return (size_t)S * num_q_heads * nparts * (head_dim + 2) * sizeof(float);
}

kv_status kv_paged_attention_decode(float* out, const void* q, const void* k_pool,
                                    const void* v_pool, const int32_t* block_tables,
                                    int32_t max_blocks, const int32_t* context_lens, int32_t S,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t num_blocks, float scale,
                                    kv_dtype dtype, int32_t partition_size,
                                    int32_t max_context_len, const int32_t* work_items,
                                    int32_t n_items, void* workspace, size_t ws_bytes,
                                    hipStream_t stream) {
  pagedkv::clear_error();
  if (pagedkv::dtype_bytes(dtype) == 0)
    return fail(KV_ERR_UNSUPPORTED, "kv_paged_attention_decode: unknown dtype");
  if (S < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks < 0 || num_blocks <= 0 ||
      max_context_len < 0)
    return fail(KV_ERR_INVALID, "kv_paged_attention_decode: bad sizes");
  if (num_q_heads % num_kv_heads != 0)
    return fail(KV_ERR_UNSUPPORTED, "kv_paged_attention_decode: query heads %d not a multiple of KV heads %d",
                num_q_heads, num_kv_heads);
  if (block_size != kBlock)
    return fail(KV_ERR_UNSUPPORTED, "kv_paged_attention_decode: block_size %d (only 16)", block_size);
  if (head_dim != 64 && head_dim != 128)
    return fail(KV_ERR_UNSUPPORTED, "kv_paged_attention_decode: head_dim %d (64 or 128)", head_dim);
  const int32_t G = num_q_heads / num_kv_heads;
  if (G > 16) return fail(KV_ERR_UNSUPPORTED, "kv_paged_attention_decode: group size %d > 16", G);
  const int32_t P = effective_partition(partition_size);
  if (P < kBlock || P > kMaxPartition || P % kBlock != 0)
    return fail(KV_ERR_INVALID, "kv_paged_attention_decode: partition_size %d", partition_size);
  if (S == 0) return KV_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens)
    return fail(KV_ERR_INVALID, "kv_paged_attention_decode: null pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(KV_ERR_INVALID, "kv_paged_attention_decode: out/q/pools must be 16-byte aligned");
  const int64_t nparts = ceil_div64(max_context_len, P) < 1 ? 1 : ceil_div64(max_context_len, P);
  const size_t need = kv_paged_attention_workspace_bytes(S, num_q_heads, num_kv_heads, head_dim,
                                                         max_context_len, partition_size);
  if (need > 0 && (!workspace || ws_bytes < need || !aligned16(workspace)))
    return fail(KV_ERR_INVALID, "kv_paged_attention_decode: workspace of %zu bytes needed (got %zu)",
                need, ws_bytes);
  if (work_items && n_items <= 0)
    return fail(KV_ERR_INVALID, "kv_paged_attention_decode: work plan with %d items", n_items);
  const int64_t n_units = work_items ? (int64_t)n_items * num_kv_heads
                                     : nparts * num_kv_heads * (int64_t)S;
  if (n_units > INT32_MAX)
    return fail(KV_ERR_INVALID, "kv_paged_attention_decode: too many work units");

  DecodeParams prm;
  prm.out = out;
  prm.q = q;
  prm.k_pool = k_pool;
  prm.v_pool = v_pool;
  prm.tables = block_tables;
  prm.lens = context_lens;
  prm.items = work_items;
  prm.n_units = (int32_t)n_units;
  float* ws = static_cast<float*>(workspace);
  const size_t o_elems = (size_t)S * num_q_heads * nparts * head_dim;
  prm.ws_o = need ? ws : nullptr;
  prm.ws_ml = need ? ws + o_elems : nullptr;
  prm.max_blocks = max_blocks;
  prm.S = S;
  prm.Hq = num_q_heads;
  prm.Hkv = num_kv_heads;
  prm.G = G;
  prm.num_blocks = num_blocks;
  prm.part_tokens = P;
  prm.nparts = (int32_t)nparts;
  prm.scale_log2 = scale * 1.4426950408889634f;

  kv_status st;
  const bool mfma = (dtype == KV_F16 || dtype == KV_BF16) && head_dim == 128 && G >= 2;
  if (mfma) {
    st = dtype == KV_BF16 ? launch_decode(decode_mfma_kernel<KV_BF16>, prm, stream)
                          : launch_decode(decode_mfma_kernel<KV_F16>, prm, stream);
  } else {
    const int gmax = G == 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : G <= 8 ? 8 : 16;
    if (dtype == KV_F32)
      st = head_dim == 64 ? launch_valu<KV_F32, 64>(prm, gmax, stream)
                          : launch_valu<KV_F32, 128>(prm, gmax, stream);
    else if (dtype == KV_F16)
      st = head_dim == 64 ? launch_valu<KV_F16, 64>(prm, gmax, stream)
                          : launch_valu<KV_F16, 128>(prm, 1, stream);
    else
      st = head_dim == 64 ? launch_valu<KV_BF16, 64>(prm, gmax, stream)
                          : launch_valu<KV_BF16, 128>(prm, 1, stream);
  }
  if (st != KV_OK || nparts <= 1) return st;
  const dim3 rgrid((unsigned)num_q_heads, (unsigned)S);
  if (head_dim == 128)
    hipLaunchKernelGGL(splitk_merge_kernel<128>, rgrid, dim3(128), 0, stream, out, prm.ws_o,
                       prm.ws_ml, context_lens, num_q_heads, prm.nparts, P, max_blocks);
  else
    hipLaunchKernelGGL(splitk_merge_kernel<64>, rgrid, dim3(64), 0, stream, out, prm.ws_o,
                       prm.ws_ml, context_lens, num_q_heads, prm.nparts, P, max_blocks);
  return launch_status("kv_paged_attention_decode (split-K merge)");
}

}  // extern "C"
