// Device side of pagedkv for AMD CDNA4 (gfx950), the cache-management half:
// slot mapping, the cache write (16-bit copy and fp8 quantisation), block
// copies for copy-on-write and block swaps to and from host memory.
//
// Pages cited in this file:
//   [1] "PagedAttention - how vLLM stopped wasting 80% of your GPU memory"
//       (shivam2003.com/posts/pagedattention.html)
//   [2] "PagedAttention: How vLLM Borrowed Virtual Memory to Unlock GPU
//       Serving at Scale" (fp4-site.pages.dev/system/pagedattention-vllm-deep-dive/)
//   [3] "PagedAttention and vLLM: Virtual Memory for the KV Cache" (passgenai.com)
//   [4] "What is paged attention?" (netraruntime.com/learn/paged-attention)

#include "device_common.h"

using namespace pagedkv::dev;

namespace {

// ============================================================================
// Slot mapping ([4], "How it works"): slot = table[p / B] * B + p % B.
// Entries that cannot be mapped give -1.
// ============================================================================
__device__ __forceinline__ int64_t slot_of(const int32_t* __restrict__ tables, int32_t num_rows,
                                           int32_t max_blocks, int32_t s, int32_t pos, int32_t B) {
  if (s < 0 || s >= num_rows || pos < 0 || pos / B >= max_blocks) return -1;
  const int32_t e = tables[(size_t)s * max_blocks + pos / B];
  return e >= 0 ? (int64_t)e * B + pos % B : -1;
}

__global__ void slot_mapping_kernel(const int32_t* __restrict__ tables, int32_t num_rows,
                                    int32_t max_blocks, const int32_t* __restrict__ seq_idx,
                                    const int32_t* __restrict__ pos, int32_t n, int32_t B,
                                    int64_t* __restrict__ slots) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  slots[i] = slot_of(tables, num_rows, max_blocks, seq_idx[i], pos[i], B);
}

// ============================================================================
// reshape_and_cache ([3], "The allocation lifecycle"): copy each new token's
// K and V rows (all KV heads) into its slot. One thread moves 16 bytes of K
// and 16 bytes of V; consecutive threads cover consecutive bytes of a token,
// so reads and writes are coalesced per head row.
// ============================================================================
__device__ __forceinline__ void copy_token_chunk(const uint4* __restrict__ k_new,
                                                 const uint4* __restrict__ v_new,
                                                 uint4* __restrict__ k_pool,
                                                 uint4* __restrict__ v_pool, int64_t i,
                                                 int64_t c, int64_t slot, int64_t num_slots,
                                                 int32_t Hkv, int32_t row_u4, int32_t B) {
  if (slot < 0 || slot >= num_slots) return;
  const int64_t h = c / row_u4, cc = c % row_u4;
  const int64_t blk = slot / B, off = slot % B;
  const int64_t dst = ((blk * Hkv + h) * B + off) * row_u4 + cc;
  const int64_t src = i * Hkv * row_u4 + c;
  k_pool[dst] = k_new[src];
  v_pool[dst] = v_new[src];
}

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
  copy_token_chunk(k_new, v_new, k_pool, v_pool, i, t % per_token, slots[i], num_slots, Hkv,
                   row_u4, B);
}

// Slot mapping and cache write in one launch: workgroup i handles new token
// i, computes its slot (thread 0 also records it) and copies its K/V rows.
__global__ void append_tokens_kernel(const int32_t* __restrict__ tables, int32_t num_rows,
                                     int32_t max_blocks, const int32_t* __restrict__ seq_idx,
                                     const int32_t* __restrict__ pos, int32_t B,
                                     int64_t* __restrict__ slots, const uint4* __restrict__ k_new,
                                     const uint4* __restrict__ v_new, uint4* __restrict__ k_pool,
                                     uint4* __restrict__ v_pool, int64_t num_slots, int32_t Hkv,
                                     int32_t row_u4) {
  const int64_t i = blockIdx.x;
  const int64_t slot = slot_of(tables, num_rows, max_blocks, seq_idx[i], pos[i], B);
  if (threadIdx.x == 0) slots[i] = slot;
  const int64_t per_token = (int64_t)Hkv * row_u4;
  for (int64_t c = threadIdx.x; c < per_token; c += blockDim.x)
    copy_token_chunk(k_new, v_new, k_pool, v_pool, i, c, slot, num_slots, Hkv, row_u4, B);
}

// ============================================================================
// fp8 cache write: as reshape_and_cache, but each 16-bit value is stored as
// the E4M3 code of value / scale (K and V pools have their own scales). One
// thread turns 8 values (16 bytes in, 8 bytes out) of K and of V.
// ============================================================================
template <int DT>
__global__ void reshape_and_cache_fp8_kernel(const uint4* __restrict__ k_new,
                                             const uint4* __restrict__ v_new,
                                             uint2* __restrict__ k_pool, uint2* __restrict__ v_pool,
                                             const int64_t* __restrict__ slots, int32_t n,
                                             int64_t num_slots, int32_t Hkv, int32_t row_c,
                                             int32_t B, float k_scale, float v_scale) {
  const int64_t per_token = (int64_t)Hkv * row_c;  // 8-value chunks per token
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)n * per_token) return;
  const int64_t i = t / per_token, c = t % per_token;
  const int64_t slot = slots[i];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t h = c / row_c, cc = c % row_c;
  const int64_t dst = (((slot / B) * Hkv + h) * B + slot % B) * row_c + cc;
  k_pool[dst] = e4m3x8_from16<DT>(k_new[t], k_scale);
  v_pool[dst] = e4m3x8_from16<DT>(v_new[t], v_scale);
}

// Elementwise E4M3 codes of a 16-bit buffer (n a multiple of 8).
template <int DT>
__global__ void quantize_fp8_kernel(const uint4* __restrict__ src, uint2* __restrict__ dst,
                                    int64_t n8, float scale) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = e4m3x8_from16<DT>(src[i], scale);
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

// ============================================================================
// Swap of whole blocks between the pools and host memory ([3], "The
// allocation lifecycle": under memory pressure a sequence's blocks are moved
// to host memory and brought back when it is readmitted; [1], "Preemption").
// Host layout [n][num_layers][2][block_bytes]: K then V of every layer, so
// one block's state for all layers is contiguous. The host buffer is pinned
// memory that the kernel reads or writes directly over the bus; blockIdx.x =
// list entry, blockIdx.y = layer within this launch's chunk, blockIdx.z = K
// (0) or V (1). Entries outside the pool are skipped.
// ============================================================================
__global__ void swap_blocks_kernel(CopyPools pools, const int32_t* __restrict__ ids,
                                   int32_t num_blocks, int64_t block_u4, uint4* host,
                                   int32_t num_layers, int32_t layer0, int32_t to_host) {
  const int32_t e = ids[blockIdx.x];
  if (e < 0 || e >= num_blocks) return;
  uint4* pool = (blockIdx.z == 0 ? pools.k[blockIdx.y] : pools.v[blockIdx.y]) + (int64_t)e * block_u4;
  uint4* h = host + (((int64_t)blockIdx.x * num_layers + layer0 + blockIdx.y) * 2 + blockIdx.z) *
                        block_u4;
  if (to_host) {
    for (int64_t i = threadIdx.x; i < block_u4; i += blockDim.x) h[i] = pool[i];
  } else {
    for (int64_t i = threadIdx.x; i < block_u4; i += blockDim.x) pool[i] = h[i];
  }
}

kv_status check_cache_write(const char* who, const void* k_new, const void* v_new,
                            const void* k_pool, const void* v_pool, int32_t n, int32_t num_blocks,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            kv_dtype dtype) {
  const size_t eb = pagedkv::dtype_bytes(dtype);
  if (eb == 0) return fail(KV_ERR_UNSUPPORTED, "%s: unknown dtype", who);
  if (n < 0 || num_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
    return fail(KV_ERR_INVALID, "%s: bad sizes", who);
  if ((head_dim * eb) % 16 != 0)
    return fail(KV_ERR_UNSUPPORTED, "%s: head_dim*elem must be a multiple of 16 bytes", who);
  if (n == 0) return KV_OK;
  if (!k_new || !v_new || !k_pool || !v_pool) return fail(KV_ERR_INVALID, "%s: null pointer", who);
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(KV_ERR_INVALID, "%s: pointers must be 16-byte aligned", who);
  return KV_OK;
}

kv_status swap_blocks(const char* who, void* const* k_pools, void* const* v_pools,
                      int32_t num_layers, const int32_t* block_ids, int32_t n,
                      int32_t num_blocks, size_t block_bytes, const void* host_buffer,
                      bool to_host, hipStream_t stream) {
  if (n < 0 || num_layers < 0 || num_layers > 256 || num_blocks <= 0)
    return fail(KV_ERR_INVALID, "%s: bad sizes", who);
  if (block_bytes == 0 || block_bytes % 16 != 0)
    return fail(KV_ERR_INVALID, "%s: block_bytes must be a positive multiple of 16", who);
  if (n == 0 || num_layers == 0) return KV_OK;
  if (!k_pools || !v_pools || !block_ids || !host_buffer)
    return fail(KV_ERR_INVALID, "%s: null pointer", who);
  if (!aligned16(host_buffer)) return fail(KV_ERR_INVALID, "%s: host buffer must be 16-byte aligned", who);
  for (int32_t i = 0; i < num_layers; ++i)
    if (!k_pools[i] || !v_pools[i] || !aligned16(k_pools[i]) || !aligned16(v_pools[i]))
      return fail(KV_ERR_INVALID, "%s: layer %d pool null or misaligned", who, i);
  void* dev_host = nullptr;
  if (hipHostGetDevicePointer(&dev_host, const_cast<void*>(host_buffer), 0) != hipSuccess ||
      !dev_host) {
    (void)hipGetLastError();  // leave no sticky error behind
    return fail(KV_ERR_INVALID, "%s: host buffer is not pinned host memory", who);
  }
  for (int32_t l0 = 0; l0 < num_layers; l0 += kCopyLayers) {
    CopyPools cp{};
    const int32_t nl = num_layers - l0 < kCopyLayers ? num_layers - l0 : kCopyLayers;
    for (int32_t i = 0; i < nl; ++i) {
      cp.k[i] = static_cast<uint4*>(k_pools[l0 + i]);
      cp.v[i] = static_cast<uint4*>(v_pools[l0 + i]);
    }
    hipLaunchKernelGGL(swap_blocks_kernel, dim3(n, nl, 2), dim3(256), 0, stream, cp, block_ids,
                       num_blocks, (int64_t)(block_bytes / 16), static_cast<uint4*>(dev_host),
                       num_layers, l0, to_host ? 1 : 0);
    kv_status st = launch_status(who);
    if (st != KV_OK) return st;
  }
  return KV_OK;
}

}  // namespace

// HBM read ceiling for the measurements: every workgroup streams 16-byte
// chunks of the buffer with non-temporal loads (the decode kernels' K/V load
// policy) in a grid-stride loop and folds them into one word per thread, and
// thread 0 stores its word per workgroup so the loads are not dead code.
constexpr int kProbeThreads = 256;
__global__ __launch_bounds__(kProbeThreads) void hbm_read_probe_kernel(const uint4* __restrict__ src,
                                                                       int64_t n16, uint32_t* sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  for (int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n16; i += stride) {
    const uint4 v = load_kv<true>(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

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
  kv_status st = check_cache_write("kv_reshape_and_cache", k_new, v_new, k_pool, v_pool, n,
                                   num_blocks, num_kv_heads, head_dim, block_size, dtype);
  if (st != KV_OK || n == 0) return st;
  if (!slots) return fail(KV_ERR_INVALID, "kv_reshape_and_cache: null pointer");
  const int32_t row_u4 = (int32_t)(head_dim * pagedkv::dtype_bytes(dtype) / 16);
  const int64_t total = (int64_t)n * num_kv_heads * row_u4;
  const int64_t blocks = ceil_div64(total, 256);
  if (blocks > INT32_MAX) return fail(KV_ERR_INVALID, "kv_reshape_and_cache: too many tokens");
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                     static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool), slots, n,
                     (int64_t)num_blocks * block_size, num_kv_heads, row_u4, block_size);
  return launch_status("kv_reshape_and_cache");
}

kv_status kv_append_tokens(const int32_t* tables, int32_t num_rows, int32_t max_blocks,
                           const int32_t* seq_idx, const int32_t* pos, int32_t n,
                           const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                           int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, kv_dtype dtype, int64_t* slots,
                           hipStream_t stream) {
  pagedkv::clear_error();
  if (num_rows < 0 || max_blocks < 0)
    return fail(KV_ERR_INVALID, "kv_append_tokens: negative size");
  kv_status st = check_cache_write("kv_append_tokens", k_new, v_new, k_pool, v_pool, n,
                                   num_blocks, num_kv_heads, head_dim, block_size, dtype);
  if (st != KV_OK || n == 0) return st;
  if (!tables || !seq_idx || !pos || !slots)
    return fail(KV_ERR_INVALID, "kv_append_tokens: null pointer");
  const int32_t row_u4 = (int32_t)(head_dim * pagedkv::dtype_bytes(dtype) / 16);
  hipLaunchKernelGGL(append_tokens_kernel, dim3((unsigned)n), dim3(64), 0, stream, tables,
                     num_rows, max_blocks, seq_idx, pos, block_size, slots,
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                     static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool),
                     (int64_t)num_blocks * block_size, num_kv_heads, row_u4);
  return launch_status("kv_append_tokens");
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

kv_status kv_swap_out_blocks(void* const* k_pools, void* const* v_pools, int32_t num_layers,
                             const int32_t* block_ids, int32_t n, int32_t num_blocks,
                             size_t block_bytes, void* host_buffer, hipStream_t stream) {
  pagedkv::clear_error();
  return swap_blocks("kv_swap_out_blocks", k_pools, v_pools, num_layers, block_ids, n,
                     num_blocks, block_bytes, host_buffer, true, stream);
}

kv_status kv_swap_in_blocks(void* const* k_pools, void* const* v_pools, int32_t num_layers,
                            const int32_t* block_ids, int32_t n, int32_t num_blocks,
                            size_t block_bytes, const void* host_buffer, hipStream_t stream) {
  pagedkv::clear_error();
  return swap_blocks("kv_swap_in_blocks", k_pools, v_pools, num_layers, block_ids, n,
                     num_blocks, block_bytes, host_buffer, false, stream);
}

kv_status kv_reshape_and_cache_fp8(const void* k_new, const void* v_new, void* k_pool,
                                   void* v_pool, const int64_t* slots, int32_t n,
                                   int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, kv_dtype dtype, float k_scale,
                                   float v_scale, hipStream_t stream) {
  pagedkv::clear_error();
  const char* who = "kv_reshape_and_cache_fp8";
  if (dtype != KV_F16 && dtype != KV_BF16)
    return fail(KV_ERR_UNSUPPORTED, "%s: new tokens must be f16 or bf16", who);
  if (!(k_scale > 0.0f) || !(v_scale > 0.0f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(KV_ERR_INVALID, "%s: scales must be finite and > 0", who);
  kv_status st = check_cache_write(who, k_new, v_new, k_pool, v_pool, n, num_blocks, num_kv_heads,
                                   head_dim, block_size, KV_FP8_E4M3);
  if (st != KV_OK || n == 0) return st;
  if (!slots) return fail(KV_ERR_INVALID, "%s: null pointer", who);
  const int32_t row_c = head_dim / 8;
  const int64_t total = (int64_t)n * num_kv_heads * row_c;
  const int64_t blocks = ceil_div64(total, 256);
  if (blocks > INT32_MAX) return fail(KV_ERR_INVALID, "%s: too many tokens", who);
  auto kern = dtype == KV_BF16 ? reshape_and_cache_fp8_kernel<KV_BF16>
                               : reshape_and_cache_fp8_kernel<KV_F16>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                     static_cast<uint2*>(k_pool), static_cast<uint2*>(v_pool), slots, n,
                     (int64_t)num_blocks * block_size, num_kv_heads, row_c, block_size, k_scale,
                     v_scale);
  return launch_status(who);
}

kv_status kv_quantize_fp8(const void* src, void* dst, int64_t n, kv_dtype dtype, float scale,
                          hipStream_t stream) {
  pagedkv::clear_error();
  const char* who = "kv_quantize_fp8";
  if (dtype != KV_F16 && dtype != KV_BF16)
    return fail(KV_ERR_UNSUPPORTED, "%s: source must be f16 or bf16", who);
  if (n < 0 || n % 8 != 0) return fail(KV_ERR_INVALID, "%s: n must be a multiple of 8", who);
  if (!(scale > 0.0f) || !std::isfinite(scale))
    return fail(KV_ERR_INVALID, "%s: scale must be finite and > 0", who);
  if (n == 0) return KV_OK;
  if (!src || !dst || !aligned16(src) || (reinterpret_cast<uintptr_t>(dst) & 7u))
    return fail(KV_ERR_INVALID, "%s: null or misaligned pointer", who);
  const int64_t n8 = n / 8;
  const int64_t blocks = ceil_div64(n8, 256) < 65536 ? ceil_div64(n8, 256) : 65536;
  auto kern = dtype == KV_BF16 ? quantize_fp8_kernel<KV_BF16> : quantize_fp8_kernel<KV_F16>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint4*>(src), static_cast<uint2*>(dst), n8, scale);
  return launch_status(who);
}

kv_status kv_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                            hipStream_t stream) {
  pagedkv::clear_error();
  const char* who = "kv_hbm_read_probe";
  if (bytes % 16 != 0 || workgroups <= 0)
    return fail(KV_ERR_INVALID, "%s: bytes a multiple of 16, workgroups > 0", who);
  if (bytes == 0) return KV_OK;
  if (!src || !sink || !aligned16(src)) return fail(KV_ERR_INVALID, "%s: null or misaligned", who);
  hipLaunchKernelGGL(hbm_read_probe_kernel, dim3((unsigned)workgroups), dim3(kProbeThreads), 0,
                     stream, static_cast<const uint4*>(src), (int64_t)(bytes / 16), sink);
  return launch_status(who);
}

}  // extern "C"
