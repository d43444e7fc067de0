// Device side of pagedkv for AMD CDNA4 (gfx950), the attention half: paged
// decode attention over 16-bit or fp8 pools, with the new token's cache write
// fused in, and the split-K merge.
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

#include <mutex>

#include "decode_kernels.h"

using namespace pagedkv::dev;
using namespace pagedkv::decode;

namespace pagedkv {
namespace decode {
// compiled in decode_variants.hip, one object per (block size, load policy)
PAGEDKV_DECODE_LAUNCHERS(extern, 8, false)
PAGEDKV_DECODE_LAUNCHERS(extern, 8, true)
PAGEDKV_DECODE_LAUNCHERS(extern, 16, false)
PAGEDKV_DECODE_LAUNCHERS(extern, 16, true)
PAGEDKV_DECODE_LAUNCHERS(extern, 32, false)
PAGEDKV_DECODE_LAUNCHERS(extern, 32, true)
}  // namespace decode
}  // namespace pagedkv

namespace {

// The decode kernel for a block size and load policy.
template <bool NT>
kv_status launch_for_block_size(const DecodeParams& prm, kv_dtype dtype, int head_dim, int G,
                                bool kv8, hipStream_t stream) {
  const int bs = prm.block_size;
  if (kv8)
    return bs == 8    ? launch_decode_kernel_fp8<8, NT>(prm, dtype, head_dim, G, stream)
           : bs == 16 ? launch_decode_kernel_fp8<16, NT>(prm, dtype, head_dim, G, stream)
                      : launch_decode_kernel_fp8<32, NT>(prm, dtype, head_dim, G, stream);
  return bs == 8    ? launch_decode_kernel<8, NT>(prm, dtype, head_dim, G, stream)
         : bs == 16 ? launch_decode_kernel<16, NT>(prm, dtype, head_dim, G, stream)
                    : launch_decode_kernel<32, NT>(prm, dtype, head_dim, G, stream);
}

// ---- the split-K partials of kv_paged_attention_decode_append_noalloc -------
// Callers that cannot allocate device memory get the library's own buffer: a
// file-scope device array, one copy per GPU, held until the process ends.
// Host code never passes the array's name to a kernel (in host code it stands
// for a host-side shadow, not the device memory); it asks the runtime for the
// array's address on the current device once and keeps it per device.
constexpr size_t kNoAllocScratchBytes = KV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device.
kv_status scratch_on_current_device(void** out, const char* who) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KV_ERR_HIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(KV_ERR_UNSUPPORTED, "%s: device %d (at most %d devices)", who, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(KV_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", who, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KV_OK;
}

}  // namespace

extern "C" {

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

namespace {

// Shared body of the decode entry points; k_new/v_new/slots are NULL for a
// plain decode and set for the fused cache write.
// The shared-prefix step's prefix pass ([1] "Memory sharing": positions every
// sequence reaches through the same blocks): attention of all S queries over
// the first `tokens` positions, in `parts` key ranges (outputs o, log2
// denominators lse); the decode kernels then cover each sequence's tail.
struct SharedPrefix {
  int32_t tokens, parts;
  float* o;
  float* lse;
};

kv_status decode_impl(float* out, const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, int32_t max_blocks,
                      const int32_t* context_lens, int32_t S, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t num_blocks, float scale, kv_dtype dtype, int32_t partition_size,
                      int32_t max_context_len, const int32_t* work_items, int32_t n_items,
                      void* workspace, size_t ws_bytes, const void* k_new, const void* v_new,
                      int64_t* slots, kv_load_policy load_policy, hipStream_t stream,
                      bool kv8 = false,
                      float k_scale = 1.0f, float v_scale = 1.0f,
                      const SharedPrefix* pre = nullptr) {
  if (pagedkv::dtype_bytes(dtype) == 0)
    return fail(KV_ERR_UNSUPPORTED, "kv_paged_attention_decode: unknown dtype");
  if (load_policy != KV_LOADS_STREAM && load_policy != KV_LOADS_CACHED)
    return fail(KV_ERR_INVALID, "kv_paged_attention_decode: unknown load policy %d",
                (int)load_policy);
  if (dtype == KV_FP8_E4M3)
    return fail(KV_ERR_UNSUPPORTED, "kv_paged_attention_decode: an fp8 cache goes through the "
                                    "_fp8 entry points (dtype is the query's type)");
  if (kv8) {
    if (dtype != KV_F16 && dtype != KV_BF16)
      return fail(KV_ERR_UNSUPPORTED, "kv_paged_attention_decode_fp8: queries must be f16 or bf16");
    if (head_dim != 64 && head_dim != 128)
      return fail(KV_ERR_UNSUPPORTED, "kv_paged_attention_decode_fp8: head_dim %d (64 or 128)",
                  head_dim);
    if (!(k_scale > 0.0f) || !(v_scale > 0.0f) || !std::isfinite(k_scale) ||
        !std::isfinite(v_scale))
      return fail(KV_ERR_INVALID, "kv_paged_attention_decode_fp8: scales must be finite and > 0");
  }
  if (S < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks < 0 || num_blocks <= 0 ||
      max_context_len < 0)
    return fail(KV_ERR_INVALID, "kv_paged_attention_decode: bad sizes");
  if (num_q_heads % num_kv_heads != 0)
    return fail(KV_ERR_UNSUPPORTED, "kv_paged_attention_decode: query heads %d not a multiple of KV heads %d",
                num_q_heads, num_kv_heads);
  if (block_size != 8 && block_size != 16 && block_size != 32)
    return fail(KV_ERR_UNSUPPORTED, "kv_paged_attention_decode: block_size %d (8, 16 or 32)",
                block_size);
  if (head_dim != 64 && head_dim != 128)
    return fail(KV_ERR_UNSUPPORTED, "kv_paged_attention_decode: head_dim %d (64 or 128)", head_dim);
  const int32_t G = num_q_heads / num_kv_heads;
  if (G > 16) return fail(KV_ERR_UNSUPPORTED, "kv_paged_attention_decode: group size %d > 16", G);
  const int32_t P = effective_partition(partition_size);
  if (P < kTile || P > kMaxPartition || P % kTile != 0 || P % block_size != 0)
    return fail(KV_ERR_INVALID,
                "kv_paged_attention_decode: partition_size %d (a multiple of 16 and of the block "
                "size, at most 1024 tokens)", partition_size);
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

  DecodeParams prm = {};  // skip_tokens 0, no prefix unless set below
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
  if (kv8) prm.scale_log2 *= k_scale;
  prm.k_scale = k_scale;
  prm.v_scale = v_scale;
  prm.k_new = k_new;
  prm.v_new = v_new;
  prm.k_pool_w = const_cast<void*>(k_pool);
  prm.v_pool_w = const_cast<void*>(v_pool);
  prm.slots = slots;
  prm.block_size = block_size;
  if (pre) {
    // the prefix pass first: the decode kernels fold its results into the outputs
    const kv_status ps = pagedkv::shared_prefix_attention(
        pre->o, pre->lse, q, k_pool, v_pool, block_tables, max_blocks, S, num_q_heads,
        num_kv_heads, block_size, num_blocks, scale, dtype, pre->tokens, kv8, k_scale, v_scale,
        stream);
    if (ps != KV_OK) return ps;
    prm.skip_tokens = pre->tokens;
    prm.pre_o = pre->o;
    prm.pre_lse = pre->lse;
    prm.pre_parts = pre->parts;
  }
  const kv_status st = load_policy == KV_LOADS_CACHED
                           ? launch_for_block_size<false>(prm, dtype, head_dim, G, kv8, stream)
                           : launch_for_block_size<true>(prm, dtype, head_dim, G, kv8, stream);
  if (st != KV_OK || nparts <= 1) return st;
  const dim3 mgrid((unsigned)((int64_t)S * num_kv_heads));
  if (pre)
    hipLaunchKernelGGL((splitk_merge_kernel<128, true>), mgrid, dim3(kMergeThreads), 0, stream, prm);
  else if (head_dim == 128)
    hipLaunchKernelGGL((splitk_merge_kernel<128, false>), mgrid, dim3(kMergeThreads), 0, stream, prm);
  else
    hipLaunchKernelGGL((splitk_merge_kernel<64, false>), mgrid, dim3(kMergeThreads), 0, stream, prm);
  return launch_status("kv_paged_attention_decode (split-K merge)");
}

}  // namespace

kv_status kv_paged_attention_decode(float* out, const void* q, const void* k_pool,
                                    const void* v_pool, const int32_t* block_tables,
                                    int32_t max_blocks, const int32_t* context_lens, int32_t S,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t num_blocks, float scale,
                                    kv_dtype dtype, int32_t partition_size,
                                    int32_t max_context_len, const int32_t* work_items,
                                    int32_t n_items, void* workspace, size_t ws_bytes,
                                    kv_load_policy load_policy, hipStream_t stream) {
  pagedkv::clear_error();
  return decode_impl(out, q, k_pool, v_pool, block_tables, max_blocks, context_lens, S,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                     partition_size, max_context_len, work_items, n_items, workspace, ws_bytes,
                     nullptr, nullptr, nullptr, load_policy, stream);
}

kv_status kv_paged_attention_decode_append(
    float* out, const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
    const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t S,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, float scale, kv_dtype dtype, int32_t partition_size,
    int32_t max_context_len, const int32_t* work_items, int32_t n_items, void* workspace,
    size_t ws_bytes, int64_t* slots, kv_load_policy load_policy, hipStream_t stream) {
  pagedkv::clear_error();
  if (S > 0) {
    if (!k_new || !v_new || !slots)
      return fail(KV_ERR_INVALID, "kv_paged_attention_decode_append: null pointer");
    if (!aligned16(k_new) || !aligned16(v_new))
      return fail(KV_ERR_INVALID, "kv_paged_attention_decode_append: k_new/v_new must be 16-byte aligned");
  }
  return decode_impl(out, q, k_pool, v_pool, block_tables, max_blocks, context_lens, S,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                     partition_size, max_context_len, work_items, n_items, workspace, ws_bytes,
                     k_new, v_new, slots, load_policy, stream);
}

kv_status kv_paged_attention_decode_append_noalloc(
    float* out, const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
    const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t S,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, float scale, kv_dtype dtype, int32_t partition_size,
    int32_t max_context_len, const int32_t* work_items, int32_t n_items, int64_t* slots,
    kv_load_policy load_policy, hipStream_t stream) {
  pagedkv::clear_error();
  const char* who = "kv_paged_attention_decode_append_noalloc";
  const size_t need = kv_paged_attention_workspace_bytes(S, num_q_heads, num_kv_heads, head_dim,
                                                         max_context_len, partition_size);
  if (need > kNoAllocScratchBytes)
    return fail(KV_ERR_INVALID,
                "%s: these sizes need %zu bytes of split-K partials and the built-in buffer "
                "holds %zu; use kv_paged_attention_decode_append with a workspace",
                who, need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0 && S > 0) {
    const kv_status st = scratch_on_current_device(&ws, who);
    if (st != KV_OK) return st;
  }
  // the decode writes every partial before the merge reads it: nothing to clear
  return kv_paged_attention_decode_append(out, q, k_new, v_new, k_pool, v_pool, block_tables,
                                          max_blocks, context_lens, S, num_q_heads, num_kv_heads,
                                          head_dim, block_size, num_blocks, scale, dtype,
                                          partition_size, max_context_len, work_items, n_items,
                                          ws, ws ? kNoAllocScratchBytes : 0, slots, load_policy,
                                          stream);
}

size_t kv_paged_attention_shared_aux_bytes(int32_t S, int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t shared_tokens) {
  int32_t part_keys = 0;
  const int32_t parts =
      pagedkv::shared_prefix_parts(S, num_q_heads, num_kv_heads, shared_tokens, &part_keys);
  if (parts <= 0 || head_dim <= 0) return 0;
  // per prefix range its outputs, then per range its denominators
  return (size_t)parts * (head_dim + 1) * S * num_q_heads * sizeof(float);
}

namespace {

// Both shared-prefix entry points: checks, then decode_impl with the prefix.
kv_status shared_impl(const char* who, float* out, const void* q, const void* k_new,
                      const void* v_new, void* k_pool, void* v_pool, const int32_t* block_tables,
                      int32_t max_blocks, const int32_t* context_lens, int32_t S,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, float scale, kv_dtype dtype,
                      int32_t partition_size, int32_t shared_tokens, int32_t max_tail_len,
                      const int32_t* work_items, int32_t n_items, void* workspace,
                      size_t ws_bytes, float* aux, size_t aux_bytes, int64_t* slots,
                      kv_load_policy load_policy, hipStream_t stream, bool kv8, float k_scale,
                      float v_scale) {
  if (dtype != KV_F16 && dtype != KV_BF16)
    return fail(KV_ERR_UNSUPPORTED, "%s: dtype must be f16 or bf16", who);
  if (head_dim != 128) return fail(KV_ERR_UNSUPPORTED, "%s: head_dim %d (128)", who, head_dim);
  if (block_size != 8 && block_size != 16 && block_size != 32)
    return fail(KV_ERR_UNSUPPORTED, "%s: block_size %d (8, 16 or 32)", who, block_size);
  if (shared_tokens <= 0 || shared_tokens % block_size != 0 ||
      shared_tokens / block_size > max_blocks)
    return fail(KV_ERR_INVALID, "%s: shared_tokens %d (whole blocks within the table)", who,
                shared_tokens);
  if (shared_tokens > KV_SHARED_PREFIX_MAX_TOKENS)
    return fail(KV_ERR_UNSUPPORTED, "%s: shared_tokens %d (at most %d)", who, shared_tokens,
                KV_SHARED_PREFIX_MAX_TOKENS);
  if (num_kv_heads > 0 && num_q_heads % num_kv_heads == 0 && num_q_heads / num_kv_heads > 16)
    return fail(KV_ERR_UNSUPPORTED, "%s: group size %d > 16", who, num_q_heads / num_kv_heads);
  if (kv8 && (!(k_scale > 0.0f) || !(v_scale > 0.0f) || !std::isfinite(k_scale) ||
              !std::isfinite(v_scale)))
    return fail(KV_ERR_INVALID, "%s: scales must be finite and > 0", who);
  if (S < 0) return fail(KV_ERR_INVALID, "%s: bad sizes", who);
  if (S == 0) return KV_OK;
  if (!k_new || !v_new || !slots || !aux)
    return fail(KV_ERR_INVALID, "%s: null pointer", who);
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(aux))
    return fail(KV_ERR_INVALID, "%s: k_new/v_new/aux must be 16-byte aligned", who);
  int32_t part_keys = 0;
  const int32_t parts =
      pagedkv::shared_prefix_parts(S, num_q_heads, num_kv_heads, shared_tokens, &part_keys);
  if (parts <= 0) return fail(KV_ERR_INVALID, "%s: bad head counts", who);
  const size_t need =
      kv_paged_attention_shared_aux_bytes(S, num_q_heads, num_kv_heads, head_dim, shared_tokens);
  if (aux_bytes < need)
    return fail(KV_ERR_INVALID, "%s: aux of %zu bytes needed (got %zu)", who, need, aux_bytes);
  const SharedPrefix pre = {shared_tokens, parts, aux,
                            aux + (size_t)parts * S * num_q_heads * head_dim};
  // checks every other argument, then the prefix pass, then the tails
  return decode_impl(out, q, k_pool, v_pool, block_tables, max_blocks, context_lens, S,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                     partition_size, max_tail_len, work_items, n_items, workspace, ws_bytes, k_new,
                     v_new, slots, load_policy, stream, kv8, k_scale, v_scale, &pre);
}

}  // namespace

kv_status kv_paged_attention_decode_append_shared(
    float* out, const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
    const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t S,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, float scale, kv_dtype dtype, int32_t partition_size,
    int32_t shared_tokens, int32_t max_tail_len, const int32_t* work_items, int32_t n_items,
    void* workspace, size_t ws_bytes, float* aux, size_t aux_bytes, int64_t* slots,
    kv_load_policy load_policy, hipStream_t stream) {
  pagedkv::clear_error();
  return shared_impl("kv_paged_attention_decode_append_shared", out, q, k_new, v_new, k_pool,
                     v_pool, block_tables, max_blocks, context_lens, S, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, scale, dtype, partition_size,
                     shared_tokens, max_tail_len, work_items, n_items, workspace, ws_bytes, aux,
                     aux_bytes, slots, load_policy, stream, false, 1.0f, 1.0f);
}

kv_status kv_paged_attention_decode_append_shared_fp8(
    float* out, const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
    const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t S,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, float scale, kv_dtype dtype, float k_scale, float v_scale,
    int32_t partition_size, int32_t shared_tokens, int32_t max_tail_len,
    const int32_t* work_items, int32_t n_items, void* workspace, size_t ws_bytes, float* aux,
    size_t aux_bytes, int64_t* slots, kv_load_policy load_policy, hipStream_t stream) {
  pagedkv::clear_error();
  return shared_impl("kv_paged_attention_decode_append_shared_fp8", out, q, k_new, v_new, k_pool,
                     v_pool, block_tables, max_blocks, context_lens, S, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, scale, dtype, partition_size,
                     shared_tokens, max_tail_len, work_items, n_items, workspace, ws_bytes, aux,
                     aux_bytes, slots, load_policy, stream, true, k_scale, v_scale);
}

kv_status kv_paged_attention_decode_fp8(float* out, const void* q, const void* k_pool,
                                        const void* v_pool, const int32_t* block_tables,
                                        int32_t max_blocks, const int32_t* context_lens,
                                        int32_t S, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                        float scale, kv_dtype dtype, float k_scale,
                                        float v_scale, int32_t partition_size,
                                        int32_t max_context_len, const int32_t* work_items,
                                        int32_t n_items, void* workspace, size_t ws_bytes,
                                        kv_load_policy load_policy, hipStream_t stream) {
  pagedkv::clear_error();
  return decode_impl(out, q, k_pool, v_pool, block_tables, max_blocks, context_lens, S,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                     partition_size, max_context_len, work_items, n_items, workspace, ws_bytes,
                     nullptr, nullptr, nullptr, load_policy, stream, true, k_scale, v_scale);
}

kv_status kv_paged_attention_decode_append_fp8(
    float* out, const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
    const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t S,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, float scale, kv_dtype dtype, float k_scale, float v_scale,
    int32_t partition_size, int32_t max_context_len, const int32_t* work_items, int32_t n_items,
    void* workspace, size_t ws_bytes, int64_t* slots, kv_load_policy load_policy,
    hipStream_t stream) {
  pagedkv::clear_error();
  if (S > 0) {
    if (!k_new || !v_new || !slots)
      return fail(KV_ERR_INVALID, "kv_paged_attention_decode_append_fp8: null pointer");
    if (!aligned16(k_new) || !aligned16(v_new))
      return fail(KV_ERR_INVALID,
                  "kv_paged_attention_decode_append_fp8: k_new/v_new must be 16-byte aligned");
  }
  return decode_impl(out, q, k_pool, v_pool, block_tables, max_blocks, context_lens, S,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                     partition_size, max_context_len, work_items, n_items, workspace, ws_bytes,
                     k_new, v_new, slots, load_policy, stream, true, k_scale, v_scale);
}

}  // extern "C"
