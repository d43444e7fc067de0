// Device side of pagedkv for AMD CDNA4 (gfx950): attention of a chunk of new
// query tokens per sequence over the paged cache, causal within the chunk
// (chunked prefill).
//
// Pages cited in this file:
//   [1] "PagedAttention - how vLLM stopped wasting 80% of your GPU memory"
//       (shivam2003.com/posts/pagedattention.html)
//   [2] "PagedAttention: How vLLM Borrowed Virtual Memory to Unlock GPU
//       Serving at Scale" (fp4-site.pages.dev/system/pagedattention-vllm-deep-dive/)
//   [4] "What is paged attention?" (netraruntime.com/learn/paged-attention)
//
// Chunked prefill feeds a prompt in pieces of a fixed token count ([2] "The
// Successors - SGLang's RadixAttention and Prefix Sharing"); each piece's K
// and V go into the sequence's blocks first ([2] "Walking Through the
// Lifecycle", Prefill), then every query token of the piece attends to all
// cached positions up to its own. Keys are reached through the block table
// exactly as in decode ([4] "How it works"), so the result is the attention
// of the contiguous cache ([1] "The PagedAttention kernel").
//
// Work split: one workgroup of four wave64s per (sequence, KV head, block of
// query rows). The 32-key K/V tiles of the sequence are staged once per
// workgroup in LDS (double buffered, loaded two tiles ahead) and shared by
// the four waves. Each wave owns two 16-column MFMA tiles; a column is one
// (query row, query head) pair of the KV head's group, so a group of G heads
// gives 16 / G query rows per column tile. Per key tile and column tile a
// wave forms
//   S^T[key][col] = K[key][:] . Q[col][:]         (8 x mfma 16x16x32: two
//                                                  16-key halves x 4 dim slices)
//   O^T[d][col]  += V^T[d][key] . P^T[key][col]   (16 x mfma 16x16x32: 8 dim
//                                                  slices x the weights as
//                                                  16-bit high part plus
//                                                  16-bit residual)
// with the causal rule key <= position(query) applied to the scores and an
// online softmax per column (lazy rescale, as in decode). The V^T operands
// come straight from the key-major LDS tile through gfx950's transposing
// LDS read.

#include "device_common.h"

using namespace pagedkv::dev;

namespace {

constexpr int kPfWaves = 4;        // waves per workgroup
constexpr int kPfColTiles = 2;     // 16-column MFMA tiles per wave
constexpr int kPfRowBytes = 272;   // LDS bytes per key row: 128 x 16-bit + 16 against bank conflicts
constexpr int kPfSegment = 64;     // table entries staged at once (one per lane)
constexpr int kPfKeys = 32;        // keys per LDS tile
constexpr int kPfHeadDim = 128;

struct PrefillParams {
  float* out;              // [T][Hq][D] fp32
  const void* q;           // [T][Hq][D]
  const void* k_pool;      // [num_blocks][Hkv][B][D]
  const void* v_pool;
  const int32_t* tables;   // [S][max_blocks]
  const int32_t* lens;     // [S] cached positions, the chunk included
  const int32_t* q_start;  // [S + 1] first query row of each sequence
  const int32_t* items;    // optional [n_items][2] = (sequence, query block)
  int32_t T, S, Hq, Hkv, G, tpc, rows_per_block, max_blocks, num_blocks, n_units, block_size;
  float scale_log2;  // scale * log2(e), times the K scale for an fp8 cache
  float v_scale;     // fp8 cache: the V scale, applied to the output
  // key split: each block's keys in `splits` runs of whole tiles, one
  // workgroup each, whose unnormalised results go to the workspace:
  int32_t splits;  // 1: no split, the kernel writes `out` itself
  float* ws_o;     // [splits][T][Hq][D] fp32, sum of weight x value (V scale applied)
  float* ws_ml;    // [splits][T][Hq][2] fp32: running max (log2 units) and weight sum
};

// Work unit b: (sequence, query block, KV head, key run). The KV head varies
// fastest, so a head's units share one XCD's L2, then the key run, then the
// plan's item (or, without a plan, the sequence, then the query block).
struct PfUnit {
  int s, qblk, h, run;
};
__device__ __forceinline__ PfUnit pf_unit(const PrefillParams& p, int b, int splits) {
  PfUnit u;
  u.h = b % p.Hkv;
  const int rest = b / p.Hkv;
  u.run = rest % splits;
  const int it = rest / splits;
  if (p.items) {
    u.s = p.items[2 * it];
    u.qblk = p.items[2 * it + 1];
  } else {
    u.s = it % p.S;
    u.qblk = it / p.S;
  }
  return u;
}

// Tiles per key run of a block with ntiles tiles: runs of equal length, so
// the last ones may be shorter or empty.
__device__ __forceinline__ int pf_run_tiles(int ntiles, int splits) {
  return (ntiles + splits - 1) / splits;
}

// Column tile of MFMA columns: query row of column c and whether it is live.
struct ColTile {
  int qrow;    // row of the chunk (0-based) this lane's column belongs to
  int pos;     // its position in the sequence: keys up to pos are visible
  bool live;
};

// gfx950 transposing LDS read (ds_read_b64_tr_b16). Within each group of 16
// lanes, the four 16-bit values that lane r names at its address form row r
// of a 16 x 4 matrix M; lane i receives M[4k + i/4][i%4] for k = 0..3, element
// k in the k-th 16-bit slot (lowest first).
__device__ __forceinline__ uint2 lds_read_tr16(const unsigned char* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
}

template <int DT, int BS, bool KV8, int CT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_mfma_kernel(PrefillParams p) {
  constexpr int D = kPfHeadDim;
  constexpr int kRowU4 = KV8 ? D / 16 : D / 8;  // uint4 per key row of the pools
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;

  const PfUnit un = pf_unit(p, blockIdx.x, p.splits);
  const int s = un.s, h = un.h, qblk = un.qblk;
  if (s < 0 || s >= p.S || qblk < 0) return;
  const int r_begin = p.q_start[s], r_end = p.q_start[s + 1];
  if (r_begin < 0 || r_end > p.T || r_end < r_begin) return;  // no row can be placed safely
  const int C = r_end - r_begin;
  const int row0 = qblk * p.rows_per_block;
  if (row0 >= C) return;
  const int rows = min(p.rows_per_block, C - row0);
  const int L = p.lens[s];
  float* const out = p.out;
  const float nan = __builtin_nanf("");
  if (L < C || (int64_t)L > (int64_t)p.max_blocks * BS) {
    // impossible length: the block's rows get NaN
    for (int i = tid; i < rows * p.G * (D / 4); i += blockDim.x) {
      const int rr = i / (p.G * (D / 4)), rem = i % (p.G * (D / 4));
      float* dst = out + ((size_t)(r_begin + row0 + rr) * p.Hq + (size_t)h * p.G) * D;
      reinterpret_cast<float4*>(dst)[rem] = make_float4(nan, nan, nan, nan);
    }
    return;
  }
  const int prev = L - C;
  const int nkeys = prev + row0 + rows;  // keys the block's last query sees
  const int ntiles = (nkeys + kPfKeys - 1) / kPfKeys;
  // this unit's run of tiles [jb, last]; an empty run (a short block split as
  // finely as the longest) has nothing to add and writes nothing
  const int tpr = pf_run_tiles(ntiles, p.splits);
  const int jb = un.run * tpr;
  const int last = min(ntiles, jb + tpr) - 1;
  if (jb > last) return;
  const int nblk = (nkeys + BS - 1) / BS;  // table entries in use

  // ---- columns and queries of this wave --------------------------------------
  ColTile ct[CT];
  uint4 qb[CT][4];
  const int hd = col % p.G;
#pragma unroll
  for (int t = 0; t < CT; ++t) {
    const int qr = row0 + (wave * CT + t) * p.tpc + col / p.G;
    ct[t].live = col < p.tpc * p.G && qr < row0 + rows;
    ct[t].qrow = qr;
    // a dead column sees every key (finite softmax of zero scores), never stored
    ct[t].pos = ct[t].live ? prev + qr : nkeys - 1;
    const uint4* qp = reinterpret_cast<const uint4*>(
        static_cast<const char*>(p.q) +
        (((size_t)r_begin + (ct[t].live ? qr : row0)) * p.Hq + (size_t)h * p.G +
         (ct[t].live ? hd : 0)) * D * 2);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const uint4 v = qp[kc * 4 + grp];
      qb[t][kc] = ct[t].live ? v : make_uint4(0, 0, 0, 0);
    }
  }

  // ---- block table: 64 entries at a time, one per lane -----------------------
  int staged = 0, seg = -1;
  bool bad = false;
  auto stage = [&](int sg) {
    const int b = sg * kPfSegment + lane;
    int e = 0;
    if (b < p.max_blocks) e = p.tables[(size_t)s * p.max_blocks + b];
    const bool need = b < nblk;
    const bool oob = need && (e < 0 || e >= p.num_blocks);
    bad = bad || __builtin_amdgcn_ballot_w64(oob) != 0;
    staged = (oob || !need) ? 0 : e;  // out-of-pool and unused entries read block 0
    seg = sg;
  };
  // A wave stages a group of consecutive rows of each tile: rows 4w..4w+3
  // and 16+4w..16+4w+3 (16-bit pools) or 8w..8w+7 (fp8 pools). Such a group
  // never straddles two blocks (8 tokens at least), so its block, table entry
  // and first row are wave-uniform and computed once per group on the scalar
  // unit; a lane adds a fixed offset (row within the group, 16-byte chunk).
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  constexpr int kGroupRows = KV8 ? 8 : 4;
  // uint4 index of the first row of the group starting at row r0 of tile j
  auto group_row = [&](int j, int r0) -> size_t {
    const int key = kPfKeys * j + r0;
    const int bi = key / BS, rb = key % BS;
    const int sg = bi / kPfSegment;
    if (sg != seg) stage(sg);
    const int e = __builtin_amdgcn_readlane(staged, bi % kPfSegment);
    return (((size_t)e * p.Hkv + h) * BS + rb) * kRowU4;
  };

  // ---- LDS tiles of 32 keys: [buffer][K, V][row] -----------------------------
  __shared__ __align__(16) unsigned char lds[2][2][kPfKeys * kPfRowBytes];
  // 16-bit pools: this lane moves rows gr and gr + 16 of the tile, 16-byte
  // chunk lc. fp8 pools: row gr, 16 codes from chunk lc, widened to two
  // 16-bit chunks.
  const int lc = KV8 ? (lane & 7) : (lane & 15);
  const int gr = kGroupRows * wv + (KV8 ? lane >> 3 : lane >> 4);  // tile row
  const int lane_u4 = (gr - kGroupRows * wv) * kRowU4 + lc;         // within the group
  // transposing V reads: key row 4grp + (col >> 2), dims 4 (col & 3)..+3
  const int vt_off = (4 * grp + (col >> 2)) * kPfRowBytes + 8 * (col & 3);
  const uint4* kpool = static_cast<const uint4*>(p.k_pool);
  const uint4* vpool = static_cast<const uint4*>(p.v_pool);
  auto load = [&](int j, uint4* g) {
    if constexpr (KV8) {
      const size_t r = group_row(j, kGroupRows * wv);
      g[0] = (kpool + r)[lane_u4];
      g[1] = (vpool + r)[lane_u4];
    } else {
      const size_t r0 = group_row(j, kGroupRows * wv), r1 = group_row(j, 16 + kGroupRows * wv);
      g[0] = (kpool + r0)[lane_u4];
      g[1] = (vpool + r0)[lane_u4];
      g[2] = (kpool + r1)[lane_u4];
      g[3] = (vpool + r1)[lane_u4];
    }
  };
  auto put = [&](int buf, int kv, int row, int chunk, const uint4& u) {
    *reinterpret_cast<uint4*>(&lds[buf][kv][row * kPfRowBytes + chunk * 16]) = u;
  };
  auto zero_past = [&](int j, int row, uint4 u) {
    return kPfKeys * j + row >= nkeys ? make_uint4(0, 0, 0, 0) : u;
  };
  auto store = [&](int j, const uint4* g, int buf) {
    // Rows past the visible keys may hold anything. Their scores are replaced
    // by -inf (a select, so even NaN keys drop out), but their zero weights
    // would still meet the values in the product: V rows there are stored as
    // zeros. Only a tail tile has such rows.
    const bool tail = kPfKeys * j + kPfKeys > nkeys;
    if constexpr (KV8) {
      const uint4 k0 = e4m3x8_widen<DT>(g[0].x, g[0].y), k1 = e4m3x8_widen<DT>(g[0].z, g[0].w);
      uint4 v0 = e4m3x8_widen<DT>(g[1].x, g[1].y), v1 = e4m3x8_widen<DT>(g[1].z, g[1].w);
      if (tail) {
        v0 = zero_past(j, gr, v0);
        v1 = zero_past(j, gr, v1);
      }
      put(buf, 0, gr, 2 * lc, k0);
      put(buf, 0, gr, 2 * lc + 1, k1);
      put(buf, 1, gr, 2 * lc, v0);
      put(buf, 1, gr, 2 * lc + 1, v1);
    } else {
      uint4 v0 = g[1], v1 = g[3];
      if (tail) {
        v0 = zero_past(j, gr, v0);
        v1 = zero_past(j, gr + 16, v1);
      }
      put(buf, 0, gr, lc, g[0]);
      put(buf, 1, gr, lc, v0);
      put(buf, 0, gr + 16, lc, g[2]);
      put(buf, 1, gr + 16, lc, v1);
    }
  };

  f32x4 o[CT][8];
  float m[CT], l[CT];
#pragma unroll
  for (int t = 0; t < CT; ++t) {
#pragma unroll
    for (int n = 0; n < 8; ++n) o[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the lowest finite value, not -inf: a column none of whose keys in a
    // run is visible (a later run of a split block) then gets weights
    // exp2(-inf - m) = 0 rather than NaN, and rescale factors exp2(m - new) 0
    m[t] = -3.402823466e38f;
    l[t] = 0.f;
  }
  // smallest position among the block's queries
  const int first_pos = prev + row0;

  // One 32-key tile. The score MFMAs run per 16-key half (lane: keys 4g..4g+3
  // of each half); the value MFMA takes all 32 keys at once, its reduction
  // index 8g+i standing for key 4g+i of the first half (i < 4) and key
  // 16+4g+i-4 of the second, in both operands.
  // Weights of 8 keys as the value product's B operands: 16-bit high parts
  // and 16-bit residuals w - high(w).
  auto split_weights = [&](const float* w, uint4& hi, uint4& lo) {
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hw[i] = pack2<DT>(w[2 * i], w[2 * i + 1]);
      float a, b;
      unpack2<DT>(hw[i], a, b);
      lw[i] = pack2<DT>(w[2 * i] - a, w[2 * i + 1] - b);
    }
    hi = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    lo = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  };

  auto compute = [&](int j, int buf) {
    // raw scores of every column tile first (K operands live); then per
    // column tile the softmax and the value products, so the MFMAs of one
    // tile can overlap the softmax of the next
    float x[CT][8];
    {
      uint4 ku[2][4];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
          ku[half][kc] = *reinterpret_cast<const uint4*>(
              &lds[buf][0][(16 * half + col) * kPfRowBytes + (kc * 4 + grp) * 16]);
#pragma unroll
      for (int t = 0; t < CT; ++t)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = 0; kc < 4; ++kc) st = mfma_qk<DT>(ku[half][kc], qb[t][kc], st);
#pragma unroll
          for (int r = 0; r < 4; ++r) x[t][4 * half + r] = st[r];
        }
    }
    // V operands: one transposing LDS read per 4 keys gives lane (i, g) dim
    // 16n + i of keys 4g..4g+3 (16 + 4g.. for the second read); the source
    // lane 4k + a of each 16-lane group names key row 4g + k, dims 16n + 4a..+3
    uint4 va[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const uint2 lo = lds_read_tr16(&lds[buf][1][vt_off + 32 * n]);
      const uint2 hi = lds_read_tr16(&lds[buf][1][vt_off + 32 * n + 16 * kPfRowBytes]);
      va[n] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
    const bool causal = kPfKeys * j + kPfKeys - 1 > first_pos;  // some key hidden from some query
    const float sl = p.scale_log2;  // > 0, so the maximum commutes with the scaling
    // maxima of every column tile first, and one rescale branch for all of
    // them, so the exponentials of one tile and the value products of
    // another sit in one straight-line block the scheduler can interleave
    float lm[CT];
    bool grow = false;
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      if (causal) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (kPfKeys * j + 16 * (i >> 2) + 4 * grp + (i & 3) > ct[t].pos) x[t][i] = neg_inf();
      }
      lm[t] = x[t][0];
#pragma unroll
      for (int i = 1; i < 8; ++i) lm[t] = fmaxf(lm[t], x[t][i]);
      lm[t] *= sl;
      grow = grow || lm[t] > m[t] + kRescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int t = 0; t < CT; ++t) {
        const float mn = fmaxf(m[t], column_max(lm[t]));
        const float alpha = fast_exp2(m[t] - mn);  // 0 while m is the initial value
        l[t] *= alpha;
#pragma unroll
        for (int n = 0; n < 8; ++n) o[t][n] *= alpha;
        m[t] = mn;
      }
    }
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      float pw[8];
      const float nm = -m[t];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pw[i] = fast_exp2(fmaf(x[t][i], sl, nm));  // 0 for hidden keys
        l[t] += pw[i];
      }
      uint4 ph, pl;
      split_weights(pw, ph, pl);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        o[t][n] = mfma_qk<DT>(va[n], ph, o[t][n]);
        o[t][n] = mfma_qk<DT>(va[n], pl, o[t][n]);
      }
    }
  };

  // ---- pipeline: tile t is loaded into register slot t % 2 two tiles ahead,
  // stored into LDS buffer t % 2 and computed after a barrier; loads and
  // stores past the last tile repeat the last tile (in bounds, never computed)
  uint4 g0[4], g1[4];
  load(jb, g0);
  store(jb, g0, 0);
  load(min(jb + 1, last), g1);
  load(min(jb + 2, last), g0);
  __syncthreads();
  for (int j = jb; j <= last; j += 2) {
    compute(j, 0);
    store(min(j + 1, last), g1, 1);
    load(min(j + 3, last), g1);
    __syncthreads();
    if (j + 1 > last) break;
    compute(j + 1, 1);
    store(min(j + 2, last), g0, 0);
    load(min(j + 4, last), g0);
    __syncthreads();
  }

  // ---- results: lane holds column col, dims 16n + 4grp + r (r < 4) -----------
  // Unsplit: the normalised output. Split: the run's unnormalised sum and its
  // (max, weight sum), combined by prefill_merge_kernel.
  const bool split = p.splits > 1;
#pragma unroll
  for (int t = 0; t < CT; ++t) {
    const float lt = column_sum(l[t]);
    if (!ct[t].live) continue;
    const float vs = KV8 ? p.v_scale : 1.0f;
    const float inv = split ? vs : vs / lt;
    const size_t orow = ((size_t)(split ? un.run : 0) * p.T + r_begin + ct[t].qrow) * p.Hq +
                        (size_t)h * p.G + hd;
    float* dst = (split ? p.ws_o : out) + orow * D + 4 * grp;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      float4 a = make_float4(o[t][n][0] * inv, o[t][n][1] * inv, o[t][n][2] * inv, o[t][n][3] * inv);
      if (bad) a = make_float4(nan, nan, nan, nan);
      *reinterpret_cast<float4*>(dst + 16 * n) = a;
    }
    if (split && grp == 0)
      *reinterpret_cast<float2*>(p.ws_ml + 2 * orow) =
          bad ? make_float2(nan, nan) : make_float2(m[t], lt);
  }
}

// Combines the key runs of a split launch: for each (query row, head) of a
// block, out = sum_r 2^(m_r - M) o_r / sum_r 2^(m_r - M) l_r with M = max_r m_r
// over the block's non-empty runs (the online-softmax rescale of the pages'
// partition-and-reduce, [2] "The Custom CUDA Kernel"). A NaN partial (an
// out-of-pool table entry) makes the row NaN. One workgroup per (plan item,
// query row of its block, KV head), a thread per (head of the group, 4
// dims); rows of a sequence with an impossible length were written (NaN) by
// the attention kernel and are left alone.
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillParams p) {
  constexpr int D = kPfHeadDim;
  const int rr = blockIdx.x % p.rows_per_block;  // row within the block
  const PfUnit un = pf_unit(p, blockIdx.x / p.rows_per_block, 1);
  const int s = un.s, h = un.h, qblk = un.qblk;
  if (s < 0 || s >= p.S || qblk < 0) return;
  const int r_begin = p.q_start[s], r_end = p.q_start[s + 1];
  if (r_begin < 0 || r_end > p.T || r_end < r_begin) return;
  const int C = r_end - r_begin;
  const int row0 = qblk * p.rows_per_block;
  if (row0 + rr >= C) return;
  const int rows = min(p.rows_per_block, C - row0);
  const int L = p.lens[s];
  if (L < C || (int64_t)L > (int64_t)p.max_blocks * p.block_size) return;
  const int nkeys = L - C + row0 + rows;
  const int ntiles = (nkeys + kPfKeys - 1) / kPfKeys;
  const int tpr = pf_run_tiles(ntiles, p.splits);
  const int runs = (ntiles + tpr - 1) / tpr;  // non-empty runs
  const size_t plane = (size_t)p.T * p.Hq;     // rows of one run in the workspace
  const float2* ml = reinterpret_cast<const float2*>(p.ws_ml);
  for (int i = threadIdx.x; i < p.G * (D / 4); i += blockDim.x) {
    const int g = i / (D / 4), c4 = i % (D / 4);
    const size_t orow = ((size_t)r_begin + row0 + rr) * p.Hq + (size_t)h * p.G + g;
    bool nan_seen = false;
    float M = -3.402823466e38f;
#pragma unroll 8
    for (int r = 0; r < runs; ++r) {
      const float mr = ml[r * plane + orow].x;
      nan_seen = nan_seen || __builtin_isnan(mr);
      M = fmaxf(M, mr);
    }
    float Lsum = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int r = 0; r < runs; ++r) {
      const float2 mlr = ml[r * plane + orow];
      const float w = exp2f(mlr.x - M);
      const float4 v = reinterpret_cast<const float4*>(p.ws_o + (r * plane + orow) * D)[c4];
      Lsum += w * mlr.y;
      acc.x += w * v.x;
      acc.y += w * v.y;
      acc.z += w * v.z;
      acc.w += w * v.w;
    }
    const float inv = 1.0f / Lsum;
    float4 res = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    if (nan_seen) {
      const float nanv = __builtin_nanf("");
      res = make_float4(nanv, nanv, nanv, nanv);
    }
    reinterpret_cast<float4*>(p.out + orow * D)[c4] = res;
  }
}

int32_t rows_per_block(int32_t G, int32_t col_tiles = kPfColTiles) {
  return kPfWaves * col_tiles * (16 / G);
}

template <bool KV8, int CT = kPfColTiles>
auto pick_kernel(kv_dtype dtype, int32_t block_size)
    -> decltype(&prefill_mfma_kernel<KV_BF16, 16, KV8, CT>) {
  if (dtype == KV_BF16)
    return block_size == 8    ? prefill_mfma_kernel<KV_BF16, 8, KV8, CT>
           : block_size == 16 ? prefill_mfma_kernel<KV_BF16, 16, KV8, CT>
                              : prefill_mfma_kernel<KV_BF16, 32, KV8, CT>;
  return block_size == 8    ? prefill_mfma_kernel<KV_F16, 8, KV8, CT>
         : block_size == 16 ? prefill_mfma_kernel<KV_F16, 16, KV8, CT>
                            : prefill_mfma_kernel<KV_F16, 32, KV8, CT>;
}

kv_status prefill_impl(const char* who, float* out, const void* q, const void* k_pool,
                       const void* v_pool, const int32_t* block_tables, int32_t max_blocks,
                       const int32_t* context_lens, const int32_t* query_start, int32_t S,
                       int32_t total_q, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                       kv_dtype dtype, int32_t max_query_len, const int32_t* work_items,
                       int32_t n_items, hipStream_t stream, bool kv8, float k_scale,
                       float v_scale, int32_t splits = 1, void* workspace = nullptr,
                       size_t ws_bytes = 0) {
  if (dtype != KV_F16 && dtype != KV_BF16)
    return fail(KV_ERR_UNSUPPORTED, "%s: dtype must be f16 or bf16", who);
  if (S < 0 || total_q < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks < 0 ||
      num_blocks <= 0 || max_query_len < 0)
    return fail(KV_ERR_INVALID, "%s: bad sizes", who);
  if (num_q_heads % num_kv_heads != 0)
    return fail(KV_ERR_UNSUPPORTED, "%s: query heads %d not a multiple of KV heads %d", who,
                num_q_heads, num_kv_heads);
  const int32_t G = num_q_heads / num_kv_heads;
  if (G > 16) return fail(KV_ERR_UNSUPPORTED, "%s: group size %d > 16", who, G);
  if (head_dim != kPfHeadDim)
    return fail(KV_ERR_UNSUPPORTED, "%s: head_dim %d (128)", who, head_dim);
  if (block_size != 8 && block_size != 16 && block_size != 32)
    return fail(KV_ERR_UNSUPPORTED, "%s: block_size %d (8, 16 or 32)", who, block_size);
  if (kv8 && (!(k_scale > 0.0f) || !(v_scale > 0.0f) || !std::isfinite(k_scale) ||
              !std::isfinite(v_scale)))
    return fail(KV_ERR_INVALID, "%s: scales must be finite and > 0", who);
  if (S == 0 || total_q == 0) return KV_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start)
    return fail(KV_ERR_INVALID, "%s: null pointer", who);
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(KV_ERR_INVALID, "%s: out/q/pools must be 16-byte aligned", who);
  if (work_items && n_items <= 0)
    return fail(KV_ERR_INVALID, "%s: work plan with %d items", who, n_items);
  if (splits < 1 || splits > KV_PREFILL_MAX_SPLITS)
    return fail(KV_ERR_INVALID, "%s: %d key splits (1..%d)", who, splits, KV_PREFILL_MAX_SPLITS);
  if (splits > 1) {
    const size_t need = kv_paged_attention_prefill_workspace_bytes(total_q, num_q_heads, head_dim,
                                                                   splits);
    if (!workspace || ws_bytes < need || !aligned16(workspace))
      return fail(KV_ERR_INVALID, "%s: workspace of %zu bytes needed (got %zu)", who, need,
                  workspace ? ws_bytes : (size_t)0);
  }
  const int32_t rpb = rows_per_block(G);
  const int64_t n_units = work_items ? (int64_t)n_items * num_kv_heads
                                     : (int64_t)S * num_kv_heads * ceil_div64(max_query_len, rpb);
  if (n_units * std::max<int64_t>(splits, rpb) > INT32_MAX)
    return fail(KV_ERR_INVALID, "%s: too many work units", who);
  if (n_units == 0) return KV_OK;

  PrefillParams prm = {};  // shared_len 0, no lse: the chunked-prefill mode
  prm.out = out;
  prm.q = q;
  prm.k_pool = k_pool;
  prm.v_pool = v_pool;
  prm.tables = block_tables;
  prm.lens = context_lens;
  prm.q_start = query_start;
  prm.items = work_items;
  prm.T = total_q;
  prm.S = S;
  prm.Hq = num_q_heads;
  prm.Hkv = num_kv_heads;
  prm.G = G;
  prm.tpc = 16 / G;
  prm.rows_per_block = rpb;
  prm.max_blocks = max_blocks;
  prm.num_blocks = num_blocks;
  prm.n_units = (int32_t)n_units;
  prm.scale_log2 = scale * 1.4426950408889634f * (kv8 ? k_scale : 1.0f);
  prm.v_scale = v_scale;
  prm.block_size = block_size;
  prm.splits = splits;
  if (splits > 1) {
    prm.ws_o = static_cast<float*>(workspace);
    prm.ws_ml = prm.ws_o + (size_t)splits * total_q * num_q_heads * head_dim;
  }

  auto kern = kv8 ? pick_kernel<true>(dtype, block_size) : pick_kernel<false>(dtype, block_size);
  hipLaunchKernelGGL(kern, dim3((unsigned)(n_units * splits)), dim3(kPfWaves * 64), 0, stream,
                     prm);
  if (splits > 1)
    hipLaunchKernelGGL(prefill_merge_kernel, dim3((unsigned)(n_units * rpb)), dim3(256), 0, stream,
                       prm);
  return launch_status(who);
}

}  // namespace

extern "C" {

int32_t kv_paged_attention_prefill_rows_per_item(int32_t num_q_heads, int32_t num_kv_heads) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return 0;
  const int32_t G = num_q_heads / num_kv_heads;
  return G > 16 ? 0 : rows_per_block(G);
}

kv_status kv_paged_attention_prefill(float* out, const void* q, const void* k_pool,
                                     const void* v_pool, const int32_t* block_tables,
                                     int32_t max_blocks, const int32_t* context_lens,
                                     const int32_t* query_start, int32_t S, int32_t total_q,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t block_size, int32_t num_blocks, float scale,
                                     kv_dtype dtype, int32_t max_query_len,
                                     const int32_t* work_items, int32_t n_items,
                                     hipStream_t stream) {
  pagedkv::clear_error();
  return prefill_impl("kv_paged_attention_prefill", out, q, k_pool, v_pool, block_tables,
                      max_blocks, context_lens, query_start, S, total_q, num_q_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                      max_query_len, work_items, n_items, stream, false, 1.0f, 1.0f);
}

size_t kv_paged_attention_prefill_workspace_bytes(int32_t total_q, int32_t num_q_heads,
                                                 int32_t head_dim, int32_t splits) {
  if (total_q <= 0 || num_q_heads <= 0 || head_dim <= 0 || splits <= 1) return 0;
  // per run and row: head_dim sums, then (max, weight sum), for every query head
  return (size_t)splits * total_q * num_q_heads * ((size_t)head_dim + 2) * sizeof(float);
}

kv_status kv_paged_attention_prefill_split(float* out, const void* q, const void* k_pool,
                                           const void* v_pool, const int32_t* block_tables,
                                           int32_t max_blocks, const int32_t* context_lens,
                                           const int32_t* query_start, int32_t S, int32_t total_q,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int32_t num_blocks, float scale, kv_dtype dtype,
                                           int32_t max_query_len, const int32_t* work_items,
                                           int32_t n_items, int32_t splits, void* workspace,
                                           size_t ws_bytes, hipStream_t stream) {
  pagedkv::clear_error();
  return prefill_impl("kv_paged_attention_prefill_split", out, q, k_pool, v_pool, block_tables,
                      max_blocks, context_lens, query_start, S, total_q, num_q_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                      max_query_len, work_items, n_items, stream, false, 1.0f, 1.0f, splits,
                      workspace, ws_bytes);
}

kv_status kv_paged_attention_prefill_split_fp8(
    float* out, const void* q, const void* k_pool, const void* v_pool,
    const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
    const int32_t* query_start, int32_t S, int32_t total_q, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    kv_dtype dtype, float k_scale, float v_scale, int32_t max_query_len,
    const int32_t* work_items, int32_t n_items, int32_t splits, void* workspace, size_t ws_bytes,
    hipStream_t stream) {
  pagedkv::clear_error();
  return prefill_impl("kv_paged_attention_prefill_split_fp8", out, q, k_pool, v_pool,
                      block_tables, max_blocks, context_lens, query_start, S, total_q,
                      num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                      max_query_len, work_items, n_items, stream, true, k_scale, v_scale, splits,
                      workspace, ws_bytes);
}

kv_status kv_paged_attention_prefill_fp8(float* out, const void* q, const void* k_pool,
                                         const void* v_pool, const int32_t* block_tables,
                                         int32_t max_blocks, const int32_t* context_lens,
                                         const int32_t* query_start, int32_t S, int32_t total_q,
                                         int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                         float scale, kv_dtype dtype, float k_scale,
                                         float v_scale, int32_t max_query_len,
                                         const int32_t* work_items, int32_t n_items,
                                         hipStream_t stream) {
  pagedkv::clear_error();
  return prefill_impl("kv_paged_attention_prefill_fp8", out, q, k_pool, v_pool, block_tables,
                      max_blocks, context_lens, query_start, S, total_q, num_q_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                      max_query_len, work_items, n_items, stream, true, k_scale, v_scale);
}

}  // extern "C"
