// Device side of pagedkv for AMD CDNA4 (gfx950): the prefix pass of the
// shared-prefix decode step.
//
// Pages cited in this file:
//   [1] "PagedAttention - how vLLM stopped wasting 80% of your GPU memory"
//       (shivam2003.com/posts/pagedattention.html)
//   [2] "PagedAttention: How vLLM Borrowed Virtual Memory to Unlock GPU
//       Serving at Scale" (fp4-site.pages.dev/system/pagedattention-vllm-deep-dive/)
//
// Sequences that share a prefix reach the same physical blocks through the
// same leading table entries ([1] "Memory sharing"). The shared-prefix step
// computes the attention of every sequence's decode query over those
// positions once for the whole batch, here, and each sequence's own tail in
// the decode kernels, which fold this pass's results into their outputs with
// the log-sum-exp rule of the split-K merge ([2] "The Custom CUDA Kernel").
//
// Work split: one workgroup of W wave64s per (key range, 16-column tile, KV
// head). A column is one (sequence, query head) pair of the KV head's group;
// all of a workgroup's waves hold the same 16 columns and each streams its
// own contiguous slice of the range's keys, with the decode kernel's register
// layouts (K straight into the score MFMA's A operand, V regrouped with
// v_perm, weights as a 16-bit high part plus residual; an fp8 cache's codes
// are widened exactly to the query's 16-bit type as they arrive, the K scale
// folded into the scores and the V scale into the outputs). At the end the W
// (max, sum, output) states of each column are merged through LDS into one
// normalised output and log2 denominator per column and range. A range
// covers W slices, so the pass writes few partial results (four ranges on a
// 2048-position prefix with 32 sequences of 4 query heads per KV head) while
// the grid still spreads the positions over the whole chip. The KV head
// varies fastest across workgroups: with a multiple of 8 heads every
// workgroup of one head runs on one XCD, so the column tiles after the first
// find that head's prefix tiles in the XCD's L2.

#include "decode_kernels.h"

namespace pagedkv {
namespace decode {
namespace {

constexpr int kShMaxWaves = 8;        // waves per workgroup (slices per range)
constexpr int kShRing = 2;            // 16-key K/V tiles in flight per wave
constexpr int kShMinTiles = 2;        // 32-position tiles per slice, at least
constexpr int kShTargetWaves = 2048;  // waves the plan aims at over the grid
constexpr int kShMaxWaveKeys = 1024;  // a wave's table entries fit its lanes
static_assert(KV_SHARED_PREFIX_MAX_TOKENS == kMaxSharedParts * kShMaxWaves * kShMaxWaveKeys,
              "the entry point's documented limit is the plan's");

struct SharedParams {
  float* o;              // [ranges][S][Hq][D] normalised outputs of each range
  float* lse;            // [ranges][S][Hq] log2 of each range's softmax denominator
  const void* q;         // [S][Hq][D]
  const void* k_pool;    // [num_blocks][Hkv][BS][D]
  const void* v_pool;
  const int32_t* table;  // row 0 of the block tables: the shared blocks first
  int32_t shared_len, ranges, range_keys, wave_keys, col_tiles;
  int32_t S, Hq, Hkv, G, num_blocks;
  float scale_log2;      // scale * log2(e), times the K scale for an fp8 cache
  float v_scale;         // fp8 cache: multiplies the outputs (1 otherwise)
};

template <int DT, int BS, bool KV8>
__global__ __launch_bounds__(64 * kShMaxWaves) void shared_prefix_kernel(SharedParams p) {
  constexpr int D = 128;
  constexpr int kRowU4 = KV8 ? D / 16 : D / 8;  // uint4 per token row of the pools
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nwaves = (int)(blockDim.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int h = blockIdx.x % p.Hkv;
  const int ctile = (blockIdx.x / p.Hkv) % p.col_tiles;
  const int range = blockIdx.x / (p.Hkv * p.col_tiles);
  if (range >= p.ranges) return;  // the whole workgroup
  // keys [k0, k0 + nk) of this wave: its slice of the range
  const int kr1 = min(p.shared_len, (range + 1) * p.range_keys);
  const int k0 = range * p.range_keys + wave * p.wave_keys;
  const int nk = max(0, min(kr1, k0 + p.wave_keys) - k0);

  // the lane's column and its query: B operand of the score MFMA, dims
  // 32kc + 8grp .. +8 (fp8 cache: dims 16grp + 8kc .. for kc < 2 and
  // 64 + 16grp + 8(kc - 2) .. for kc >= 2, the order of the lane's two
  // 16-byte K code loads); dead columns of the last tile get zeros, never stored
  const int cidx = ctile * 16 + col;
  const bool live = cidx < p.S * p.G;
  const size_t orow = live ? (size_t)(cidx / p.G) * p.Hq + (size_t)h * p.G + cidx % p.G : 0;
  uint4 qb[4];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(static_cast<const char*>(p.q) + orow * D * 2);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const uint4 v = qp[KV8 ? (kc >> 1) * 8 + 2 * grp + (kc & 1) : kc * 4 + grp];
      qb[kc] = live ? v : make_uint4(0, 0, 0, 0);
    }
  }

  // the slice's table entries, one (two with 8-token blocks) per lane
  DecodeParams dp = {};
  dp.Hkv = p.Hkv;
  dp.num_blocks = p.num_blocks;
  bool bad = false;
  Entries staged{0, 0};
  const int nent = (nk + BS - 1) / BS;
  if (nk > 0) staged = stage_entries<BS>(dp, p.table + k0 / BS, nent, nent, lane, bad);

  f32x4 o[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = neg_inf(), l = 0.f;
  const uint4* kbase = static_cast<const uint4*>(p.k_pool);
  const int nblk = (nk + kTile - 1) / kTile;  // 16-key tiles
  const int last = nblk - 1;

  // K: row col of the tile, chunks kc*4+grp (fp8: the 16-code chunks grp and
  // 4+grp); V: rows 4grp..4grp+3, chunk col (fp8: its 8 codes). Rows past the
  // slice read its last row or row group instead (masked).
  constexpr int kKU = KV8 ? 2 : 4;
  typedef typename std::conditional<KV8, uint2, uint4>::type VRaw;
  auto load = [&](int j, uint4* ku, VRaw* vu) {
    const int lim = nk - j * kTile - 1;  // last row of tile j in the slice
    const uint4* kt = kbase + tile_row<BS>(dp, h, staged, j, min(col, lim), kRowU4);
    if constexpr (KV8) {
      const uint2* vt = static_cast<const uint2*>(p.v_pool) +
                        tile_row<BS>(dp, h, staged, j, 4 * min(grp, lim >> 2), 2 * kRowU4);
      ku[0] = kt[grp];
      ku[1] = kt[4 + grp];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) vu[jj] = vt[jj * 2 * kRowU4 + col];
    } else {
      const uint4* vt = static_cast<const uint4*>(p.v_pool) +
                        tile_row<BS>(dp, h, staged, j, 4 * min(grp, lim >> 2), kRowU4);
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) ku[kc] = kt[kc * 4 + grp];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) vu[jj] = vt[jj * kRowU4 + col];
    }
  };
  auto compute16 = [&](int jb, const uint4* ku, uint4* vu) {
    f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) st = mfma_qk<DT>(ku[kc], qb[kc], st);
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = st[r] * p.scale_log2;
    const int valid = nk - jb * kTile;  // keys of the tile in the slice (>= 1)
    if (valid < kTile) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * grp + r >= valid) {
          x[r] = neg_inf();
          vu[r] = make_uint4(0, 0, 0, 0);  // rows past the slice may hold anything
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
      pw[r] = fast_exp2(x[r] - m);  // 0 for masked keys
      l += pw[r];
    }
    const uint2 ph = weight_part<DT>(pw, 0.0f);
    const uint2 pl = weight_part<DT>(pw, 1.0f);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const uint2 a = v_column(vu, n);
      o[n] = mfma_pv<DT>(a, ph, o[n]);
      o[n] = mfma_pv<DT>(a, pl, o[n]);
    }
  };
  auto compute = [&](int jb, const uint4* ku, VRaw* vu) {
    if constexpr (KV8) {
      // the codes widened to the query's 16-bit type (exact), then as above
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

  // ring of kShRing tiles, as in the decode kernel: unconditional loads in
  // the steady state, guarded refills while draining
  if (nblk > 0) {
    uint4 kr[kShRing][kKU];
    VRaw vr[kShRing][4];
#pragma unroll
    for (int s = 0; s < kShRing; ++s) load(min(s, last), kr[s], vr[s]);
    int j = 0;
    for (; j + 2 * kShRing <= nblk; j += kShRing) {
#pragma unroll
      for (int s = 0; s < kShRing; ++s) {
        compute(j + s, kr[s], vr[s]);
        load(j + s + kShRing, kr[s], vr[s]);
      }
    }
#pragma unroll
    for (int s = 0; s < kShRing; ++s) {
      if (j + s < nblk) compute(j + s, kr[s], vr[s]);
      if (j + s + kShRing < nblk) load(j + s + kShRing, kr[s], vr[s]);
    }
#pragma unroll
    for (int s = 0; s < kShRing; ++s)
      if (j + kShRing + s < nblk) compute(j + kShRing + s, kr[s], vr[s]);
  }
  l = column_sum(l);

  // Merge the waves' states per column (softmax over the union of their key
  // slices): M = max_w m_w, L = sum_w l_w 2^(m_w - M), out = sum_w o_w 2^(m_w - M) / L.
  // A wave without keys has m = -inf, l = 0 and weight 0.
  __shared__ float sh_m[kShMaxWaves][16], sh_l[kShMaxWaves][16];
  __shared__ int sh_bad[kShMaxWaves];
  __shared__ __align__(16) float sh_o[kShMaxWaves][16 * kStageStride];
  if (grp == 0) {
    sh_m[wave][col] = m;
    sh_l[wave][col] = l;
  }
  if (lane == 0) sh_bad[wave] = bad ? 1 : 0;
  __syncthreads();
  float M = neg_inf();
  bool any_bad = false;
  for (int w = 0; w < nwaves; ++w) {
    M = fmaxf(M, sh_m[w][col]);
    any_bad = any_bad || sh_bad[w] != 0;
  }
  float L = 0.f;
  for (int w = 0; w < nwaves; ++w) L += sh_l[w][col] * fast_exp2(sh_m[w][col] - M);
  float a = fast_exp2(m - M) / L;
  if constexpr (KV8) a *= p.v_scale;
  // lane holds column col, dims 32grp + 8r + n for r < 4, n < 8
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      *reinterpret_cast<float4*>(&sh_o[wave][col * kStageStride + 32 * grp + 8 * r + 4 * hh]) =
          make_float4(o[4 * hh][r] * a, o[4 * hh + 1][r] * a, o[4 * hh + 2][r] * a,
                      o[4 * hh + 3][r] * a);
  const size_t rows = (size_t)p.S * p.Hq;
  const float nan = __builtin_nanf("");
  if (wave == 0 && grp == 0 && live)
    p.lse[(size_t)range * rows + orow] = any_bad ? nan : M + log2f(L);
  __syncthreads();
  // float4 f of the tile's 16 x 128 outputs: column f / 32, dims 4(f % 32)..
  for (int f = tid; f < 16 * (D / 4); f += blockDim.x) {
    const int c = f / (D / 4), d4 = f % (D / 4);
    const int ci = ctile * 16 + c;
    if (ci >= p.S * p.G) continue;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int w = 0; w < nwaves; ++w) {
      const float4 v = *reinterpret_cast<const float4*>(&sh_o[w][c * kStageStride + 4 * d4]);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    if (any_bad) acc = make_float4(nan, nan, nan, nan);
    const size_t row = (size_t)(ci / p.G) * p.Hq + (size_t)h * p.G + ci % p.G;
    *reinterpret_cast<float4*>(p.o + ((size_t)range * rows + row) * D + 4 * d4) = acc;
  }
}

// How the shared positions are cut: slices of wave_keys positions (a multiple
// of 32, so of every block size), waves slices per workgroup, ranges of
// waves * wave_keys positions.
struct SharedPlan {
  int32_t ranges, range_keys, wave_keys, waves, col_tiles;
};

// About two waves per SIMD over the whole grid (2,048 on the MI355X's 256
// CUs), slices of 64 to 1,024 positions, at most 8 waves per workgroup;
// longer slices when the ranges would exceed kMaxSharedParts. Zero ranges
// for invalid sizes or a prefix beyond kMaxSharedParts * 8 * 1024 positions.
// Measured on MI355X (32 sequences sharing 2,048 positions, 32/8 heads, one
// box): 256 workgroups of 8 waves on 64-position slices with 2 tiles in
// flight, 4 ranges, 22.8-22.9 us per step; 4 waves on 128-position slices
// the same; 3 or 4 tiles in flight 23.0-23.7 us; 128 workgroups (2 ranges,
// half the CUs idle) 27.2-27.3 us; 8 ranges of 2 waves 24.4-24.7 us.
SharedPlan plan_shared(int32_t S, int32_t num_q_heads, int32_t num_kv_heads, int32_t shared_len) {
  SharedPlan sp = {0, 0, 0, 0, 0};
  if (S <= 0 || num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      shared_len <= 0)
    return sp;
  const int64_t G = num_q_heads / num_kv_heads;
  if (G > 16) return sp;
  const int64_t col_tiles = ceil_div64((int64_t)S * G, 16);
  const int64_t t32 = ceil_div64(shared_len, 32);
  const int64_t max_per = kShMaxWaveKeys / 32;
  int64_t per = std::max<int64_t>(kShMinTiles,
                                  ceil_div64(t32 * col_tiles * num_kv_heads, kShTargetWaves));
  per = std::min(per, max_per);
  const int64_t wpp = ceil_div64(t32, per);  // slices per (column tile, head)
  const int64_t waves = std::min<int64_t>(kShMaxWaves, wpp);
  if (ceil_div64(wpp, waves) > kMaxSharedParts) per = ceil_div64(t32, waves * kMaxSharedParts);
  if (per > max_per) return sp;
  sp.wave_keys = (int32_t)(per * 32);
  sp.waves = (int32_t)waves;
  sp.range_keys = sp.wave_keys * sp.waves;
  sp.ranges = (int32_t)ceil_div64(shared_len, sp.range_keys);
  sp.col_tiles = (int32_t)col_tiles;
  return sp;
}

template <int DT, bool KV8>
auto pick_shared_kernel(int32_t block_size) {
  return block_size == 8 ? shared_prefix_kernel<DT, 8, KV8>
         : block_size == 16 ? shared_prefix_kernel<DT, 16, KV8>
                            : shared_prefix_kernel<DT, 32, KV8>;
}

}  // namespace
}  // namespace decode

int32_t shared_prefix_parts(int32_t S, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t shared_len, int32_t* part_keys) {
  const decode::SharedPlan sp = decode::plan_shared(S, num_q_heads, num_kv_heads, shared_len);
  *part_keys = sp.range_keys;
  return sp.ranges;
}

kv_status shared_prefix_attention(float* o, float* lse, const void* q, const void* k_pool,
                                  const void* v_pool, const int32_t* table_row0,
                                  int32_t max_blocks, int32_t S, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t block_size, int32_t num_blocks,
                                  float scale, kv_dtype dtype, int32_t shared_len, bool kv8,
                                  float k_scale, float v_scale, hipStream_t stream) {
  using namespace decode;
  const SharedPlan sp = plan_shared(S, num_q_heads, num_kv_heads, shared_len);
  if (sp.ranges <= 0) return fail(KV_ERR_INVALID, "shared prefix: bad sizes");
  if ((int64_t)shared_len > (int64_t)max_blocks * block_size)
    return fail(KV_ERR_INVALID, "shared prefix: %d positions beyond the table", shared_len);
  SharedParams prm = {};
  prm.o = o;
  prm.lse = lse;
  prm.q = q;
  prm.k_pool = k_pool;
  prm.v_pool = v_pool;
  prm.table = table_row0;
  prm.shared_len = shared_len;
  prm.ranges = sp.ranges;
  prm.range_keys = sp.range_keys;
  prm.wave_keys = sp.wave_keys;
  prm.col_tiles = sp.col_tiles;
  prm.S = S;
  prm.Hq = num_q_heads;
  prm.Hkv = num_kv_heads;
  prm.G = num_q_heads / num_kv_heads;
  prm.num_blocks = num_blocks;
  prm.scale_log2 = scale * 1.4426950408889634f * (kv8 ? k_scale : 1.0f);
  prm.v_scale = kv8 ? v_scale : 1.0f;
  const int64_t groups = (int64_t)sp.ranges * sp.col_tiles * num_kv_heads;
  if (groups > INT32_MAX) return fail(KV_ERR_INVALID, "shared prefix: too many workgroups");
  auto kern = kv8 ? (dtype == KV_BF16 ? pick_shared_kernel<KV_BF16, true>(block_size)
                                     : pick_shared_kernel<KV_F16, true>(block_size))
                  : (dtype == KV_BF16 ? pick_shared_kernel<KV_BF16, false>(block_size)
                                      : pick_shared_kernel<KV_F16, false>(block_size));
  hipLaunchKernelGGL(kern, dim3((unsigned)groups), dim3(64 * sp.waves), 0, stream, prm);
  return launch_status("kv_paged_attention_decode_append_shared (shared prefix)");
}

}  // namespace pagedkv
