// Host block manager behind the pagedkv C ABI: free list, reference counts,
// sequences, fork and copy-on-write decisions. Pure C++17, no HIP calls, so
// it builds and runs on a machine without a GPU.
//
// Pages cited in this file:
//   [1] "PagedAttention - how vLLM stopped wasting 80% of your GPU memory"
//       (shivam2003.com/posts/pagedattention.html)
//   [2] "PagedAttention: How vLLM Borrowed Virtual Memory to Unlock GPU
//       Serving at Scale" (fp4-site.pages.dev/system/pagedattention-vllm-deep-dive/)
//   [3] "PagedAttention and vLLM: Virtual Memory for the KV Cache" (passgenai.com)
//   [4] "What is paged attention?" (netraruntime.com/learn/paged-attention)
//
// Design: the free list is a vector used as a LIFO stack (pop and push are
// O(1), [4] "How it works"). Reference counts live in a flat int32 array
// indexed by block ID ([1], "Memory sharing"). Each sequence keeps its block
// table as a vector. Every mutating call validates first and mutates after,
// so a failing call changes nothing ([3], "L3": all-or-nothing). A sequence
// can be swapped out under memory pressure ([3], "The allocation lifecycle";
// [1], "Preemption"): its blocks are released and it keeps only its length
// until it is swapped back in.

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv.h"
#include "status.h"

struct kv_pool {
  kv_pool_config cfg;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> refcount;    // 0 = free
  struct Seq {
    std::vector<int32_t> blocks;
    int32_t len = 0;
    bool swapped = false;  // blocks released to the pool, contents on the host
  };
  std::unordered_map<int64_t, Seq> seqs;
  int64_t next_seq = 0;
};

namespace pagedkv {

static thread_local std::string g_last_error;

kv_status fail(kv_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

size_t dtype_bytes(kv_dtype dt) {
  switch (dt) {
    case KV_F32: return 4;
    case KV_F16: return 2;
    case KV_BF16: return 2;
    case KV_FP8_E4M3: return 1;
  }
  return 0;
}

}  // namespace pagedkv

using pagedkv::fail;

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static void set_default_order(kv_pool* p) {
  const int32_t n = p->cfg.num_blocks;
  p->free_stack.resize(n);
  // block 0 must be handed out first: it sits at the back of the stack
  for (int32_t i = 0; i < n; ++i) p->free_stack[i] = n - 1 - i;
}

extern "C" {

kv_status kv_pool_create(const kv_pool_config* cfg, kv_pool_t** out) {
  pagedkv::clear_error();
  if (!cfg || !out) return fail(KV_ERR_INVALID, "kv_pool_create: null argument");
  if (cfg->num_blocks <= 0 || cfg->block_size <= 0 || cfg->num_layers <= 0 ||
      cfg->num_kv_heads <= 0 || cfg->head_dim <= 0)
    return fail(KV_ERR_INVALID, "kv_pool_create: sizes must be positive");
  if (pagedkv::dtype_bytes(cfg->dtype) == 0)
    return fail(KV_ERR_INVALID, "kv_pool_create: unknown dtype %d", (int)cfg->dtype);
  kv_pool* p = new (std::nothrow) kv_pool();
  if (!p) return fail(KV_ERR_OOM, "kv_pool_create: host allocation failed");
  p->cfg = *cfg;
  p->refcount.assign(cfg->num_blocks, 0);
  set_default_order(p);
  *out = p;
  return KV_OK;
}

void kv_pool_destroy(kv_pool_t* pool) { delete pool; }

kv_status kv_pool_set_free_order(kv_pool_t* p, int32_t n, const int32_t* order) {
  pagedkv::clear_error();
  if (!p || !order) return fail(KV_ERR_INVALID, "kv_pool_set_free_order: null argument");
  if (n != p->cfg.num_blocks)
    return fail(KV_ERR_INVALID, "kv_pool_set_free_order: need %d entries, got %d",
                p->cfg.num_blocks, n);
  if ((int32_t)p->free_stack.size() != p->cfg.num_blocks)
    return fail(KV_ERR_STATE, "kv_pool_set_free_order: blocks are in use");
  std::vector<char> seen(n, 0);
  for (int32_t i = 0; i < n; ++i) {
    if (order[i] < 0 || order[i] >= n || seen[order[i]])
      return fail(KV_ERR_INVALID, "kv_pool_set_free_order: not a permutation at %d", i);
    seen[order[i]] = 1;
  }
  for (int32_t i = 0; i < n; ++i) p->free_stack[i] = order[n - 1 - i];
  return KV_OK;
}

size_t kv_pool_layer_bytes(const kv_pool_t* p) {
  if (!p) return 0;
  return (size_t)p->cfg.num_blocks * p->cfg.num_kv_heads * p->cfg.block_size *
         p->cfg.head_dim * pagedkv::dtype_bytes(p->cfg.dtype);
}

int64_t kv_pool_capacity_tokens(const kv_pool_t* p) {
  if (!p) return -1;
  return (int64_t)p->cfg.num_blocks * p->cfg.block_size;
}

int32_t kv_num_free_blocks(const kv_pool_t* p) {
  return p ? (int32_t)p->free_stack.size() : -1;
}

kv_status kv_block_alloc(kv_pool_t* p, int32_t n, int32_t* ids_out) {
  pagedkv::clear_error();
  if (!p || (n > 0 && !ids_out)) return fail(KV_ERR_INVALID, "kv_block_alloc: null argument");
  if (n < 0) return fail(KV_ERR_INVALID, "kv_block_alloc: negative count");
  if ((size_t)n > p->free_stack.size())
    return fail(KV_ERR_OOM, "kv_block_alloc: need %d blocks, %zu free", n, p->free_stack.size());
  for (int32_t i = 0; i < n; ++i) {
    int32_t b = p->free_stack.back();
    p->free_stack.pop_back();
    p->refcount[b] = 1;
    ids_out[i] = b;
  }
  return KV_OK;
}

// Validate that every listed block is held and, when decrementing, that no
// block would drop below zero (duplicates counted).
static kv_status check_held(const kv_pool* p, int32_t n, const int32_t* ids, bool decrement,
                            const char* who) {
  std::unordered_map<int32_t, int32_t> need;
  for (int32_t i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= p->cfg.num_blocks)
      return fail(KV_ERR_INVALID, "%s: block %d outside the pool", who, ids[i]);
    need[ids[i]] += 1;
  }
  for (auto& kv : need) {
    int32_t rc = p->refcount[kv.first];
    if (rc == 0 || (decrement && rc < kv.second))
      return fail(KV_ERR_STATE, "%s: block %d is not held", who, kv.first);
  }
  return KV_OK;
}

kv_status kv_block_incref(kv_pool_t* p, int32_t n, const int32_t* ids) {
  pagedkv::clear_error();
  if (!p || (n > 0 && !ids)) return fail(KV_ERR_INVALID, "kv_block_incref: null argument");
  if (n < 0) return fail(KV_ERR_INVALID, "kv_block_incref: negative count");
  kv_status st = check_held(p, n, ids, false, "kv_block_incref");
  if (st != KV_OK) return st;
  for (int32_t i = 0; i < n; ++i) p->refcount[ids[i]] += 1;
  return KV_OK;
}

static void decref_unchecked(kv_pool* p, int32_t n, const int32_t* ids) {
  // reverse order: the first listed block ends on top of the stack
  for (int32_t i = n - 1; i >= 0; --i) {
    int32_t b = ids[i];
    if (--p->refcount[b] == 0) p->free_stack.push_back(b);
  }
}

kv_status kv_block_free(kv_pool_t* p, int32_t n, const int32_t* ids) {
  pagedkv::clear_error();
  if (!p || (n > 0 && !ids)) return fail(KV_ERR_INVALID, "kv_block_free: null argument");
  if (n < 0) return fail(KV_ERR_INVALID, "kv_block_free: negative count");
  kv_status st = check_held(p, n, ids, true, "kv_block_free");
  if (st != KV_OK) return st;
  decref_unchecked(p, n, ids);
  return KV_OK;
}

int32_t kv_block_refcount(const kv_pool_t* p, int32_t id) {
  if (!p || id < 0 || id >= p->cfg.num_blocks) return -1;
  return p->refcount[id];
}

kv_status kv_seq_create(kv_pool_t* p, int64_t* seq_out) {
  pagedkv::clear_error();
  if (!p || !seq_out) return fail(KV_ERR_INVALID, "kv_seq_create: null argument");
  int64_t id = p->next_seq++;
  p->seqs.emplace(id, kv_pool::Seq());
  *seq_out = id;
  return KV_OK;
}

kv_status kv_seq_fork(kv_pool_t* p, int64_t parent, int64_t* child_out) {
  pagedkv::clear_error();
  if (!p || !child_out) return fail(KV_ERR_INVALID, "kv_seq_fork: null argument");
  auto it = p->seqs.find(parent);
  if (it == p->seqs.end()) return fail(KV_ERR_STATE, "kv_seq_fork: unknown sequence %lld",
                                       (long long)parent);
  if (it->second.swapped)
    return fail(KV_ERR_STATE, "kv_seq_fork: sequence %lld is swapped out", (long long)parent);
  kv_pool::Seq child = it->second;  // copy before the map may rehash
  // every block must still be held (a raw kv_block_free may have dropped it)
  kv_status st = check_held(p, (int32_t)child.blocks.size(), child.blocks.data(), false,
                            "kv_seq_fork");
  if (st != KV_OK) return st;
  for (int32_t b : child.blocks) p->refcount[b] += 1;
  int64_t id = p->next_seq++;
  p->seqs.emplace(id, std::move(child));
  *child_out = id;
  return KV_OK;
}

kv_status kv_seq_append(kv_pool_t* p, int64_t seq, int32_t n_tokens, int64_t* slots_out,
                        int32_t* cow_src, int32_t* cow_dst, int32_t* n_cow) {
  pagedkv::clear_error();
  if (!p || !cow_src || !cow_dst || !n_cow)
    return fail(KV_ERR_INVALID, "kv_seq_append: null argument");
  if (n_tokens < 0) return fail(KV_ERR_INVALID, "kv_seq_append: negative token count");
  if (n_tokens > 0 && !slots_out) return fail(KV_ERR_INVALID, "kv_seq_append: null slots_out");
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end())
    return fail(KV_ERR_STATE, "kv_seq_append: unknown sequence %lld", (long long)seq);
  kv_pool::Seq& s = it->second;
  *n_cow = 0;
  if (s.swapped)
    return fail(KV_ERR_STATE, "kv_seq_append: sequence %lld is swapped out", (long long)seq);
  if (n_tokens == 0) return KV_OK;
  const int64_t B = p->cfg.block_size;
  const int64_t t = s.len;
  if (t + n_tokens > (int64_t)INT32_MAX)
    return fail(KV_ERR_INVALID, "kv_seq_append: sequence length overflow");
  const int64_t have = ceil_div(t, B);
  const int64_t need_new = ceil_div(t + n_tokens, B) - have;
  // the first new token lands in the last block when t is not a multiple
  // of B; if that block is shared, it must be copied first ([2], CoW)
  const bool cow = (t % B != 0) && p->refcount[s.blocks.back()] > 1;
  const int64_t need = need_new + (cow ? 1 : 0);
  if (need > (int64_t)p->free_stack.size())
    return fail(KV_ERR_OOM, "kv_seq_append: need %lld blocks, %zu free", (long long)need,
                p->free_stack.size());
  if (cow) {
    int32_t src = s.blocks.back();
    int32_t dst = p->free_stack.back();
    p->free_stack.pop_back();
    p->refcount[dst] = 1;
    p->refcount[src] -= 1;  // stays >= 1: it was > 1
    s.blocks.back() = dst;
    *cow_src = src;
    *cow_dst = dst;
    *n_cow = 1;
  }
  for (int64_t i = 0; i < need_new; ++i) {
    int32_t b = p->free_stack.back();
    p->free_stack.pop_back();
    p->refcount[b] = 1;
    s.blocks.push_back(b);
  }
  for (int64_t i = 0; i < n_tokens; ++i) {
    int64_t pos = t + i;
    slots_out[i] = (int64_t)s.blocks[pos / B] * B + pos % B;
  }
  s.len = (int32_t)(t + n_tokens);
  return KV_OK;
}

kv_status kv_seq_free(kv_pool_t* p, int64_t seq) {
  pagedkv::clear_error();
  if (!p) return fail(KV_ERR_INVALID, "kv_seq_free: null pool");
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end())
    return fail(KV_ERR_STATE, "kv_seq_free: unknown sequence %lld", (long long)seq);
  const std::vector<int32_t>& bl = it->second.blocks;  // empty when swapped out
  kv_status st = check_held(p, (int32_t)bl.size(), bl.data(), true, "kv_seq_free");
  if (st != KV_OK) return st;
  decref_unchecked(p, (int32_t)bl.size(), bl.data());
  p->seqs.erase(it);
  return KV_OK;
}

kv_status kv_seq_block_table(const kv_pool_t* p, int64_t seq, int32_t cap, int32_t* ids,
                             int32_t* n) {
  pagedkv::clear_error();
  if (!p || !n) return fail(KV_ERR_INVALID, "kv_seq_block_table: null argument");
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end())
    return fail(KV_ERR_STATE, "kv_seq_block_table: unknown sequence %lld", (long long)seq);
  if (it->second.swapped)
    return fail(KV_ERR_STATE, "kv_seq_block_table: sequence %lld is swapped out", (long long)seq);
  const std::vector<int32_t>& bl = it->second.blocks;
  *n = (int32_t)bl.size();
  if (cap < (int32_t)bl.size() || (!ids && !bl.empty()))
    return fail(KV_ERR_INVALID, "kv_seq_block_table: capacity %d < %zu", cap, bl.size());
  if (!bl.empty()) std::memcpy(ids, bl.data(), bl.size() * sizeof(int32_t));
  return KV_OK;
}

int32_t kv_seq_len(const kv_pool_t* p, int64_t seq) {
  if (!p) return -1;
  auto it = p->seqs.find(seq);
  return it == p->seqs.end() ? -1 : it->second.len;
}

kv_status kv_seq_pack_tables(const kv_pool_t* p, int32_t n_seqs, const int64_t* seqs,
                             int32_t max_blocks, int32_t* tables_out, int32_t* lens_out) {
  pagedkv::clear_error();
  if (!p || (n_seqs > 0 && (!seqs || !tables_out || !lens_out)))
    return fail(KV_ERR_INVALID, "kv_seq_pack_tables: null argument");
  if (n_seqs < 0 || max_blocks < 0) return fail(KV_ERR_INVALID, "kv_seq_pack_tables: sizes");
  for (int32_t i = 0; i < n_seqs; ++i) {
    auto it = p->seqs.find(seqs[i]);
    if (it == p->seqs.end())
      return fail(KV_ERR_STATE, "kv_seq_pack_tables: unknown sequence %lld",
                  (long long)seqs[i]);
    if (it->second.swapped)
      return fail(KV_ERR_STATE, "kv_seq_pack_tables: sequence %lld is swapped out",
                  (long long)seqs[i]);
    if ((int32_t)it->second.blocks.size() > max_blocks)
      return fail(KV_ERR_INVALID, "kv_seq_pack_tables: sequence %lld needs %zu > %d entries",
                  (long long)seqs[i], it->second.blocks.size(), max_blocks);
  }
  for (int32_t i = 0; i < n_seqs; ++i) {
    const kv_pool::Seq& s = p->seqs.find(seqs[i])->second;
    int32_t* row = tables_out + (size_t)i * max_blocks;
    std::fill(row, row + max_blocks, -1);
    std::copy(s.blocks.begin(), s.blocks.end(), row);
    lens_out[i] = s.len;
  }
  return KV_OK;
}

kv_status kv_seq_swap_out(kv_pool_t* p, int64_t seq, int32_t cap, int32_t* ids_out,
                          int32_t* n) {
  pagedkv::clear_error();
  if (!p || !n) return fail(KV_ERR_INVALID, "kv_seq_swap_out: null argument");
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end())
    return fail(KV_ERR_STATE, "kv_seq_swap_out: unknown sequence %lld", (long long)seq);
  kv_pool::Seq& s = it->second;
  if (s.swapped)
    return fail(KV_ERR_STATE, "kv_seq_swap_out: sequence %lld is already swapped out",
                (long long)seq);
  *n = (int32_t)s.blocks.size();
  if (cap < *n || (!ids_out && *n > 0))
    return fail(KV_ERR_INVALID, "kv_seq_swap_out: capacity %d < %d", cap, *n);
  kv_status st = check_held(p, *n, s.blocks.data(), true, "kv_seq_swap_out");
  if (st != KV_OK) return st;
  if (*n > 0) std::memcpy(ids_out, s.blocks.data(), (size_t)*n * sizeof(int32_t));
  decref_unchecked(p, *n, s.blocks.data());
  s.blocks.clear();
  s.swapped = true;
  return KV_OK;
}

kv_status kv_seq_swap_in(kv_pool_t* p, int64_t seq, int32_t cap, int32_t* ids_out, int32_t* n) {
  pagedkv::clear_error();
  if (!p || !n) return fail(KV_ERR_INVALID, "kv_seq_swap_in: null argument");
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end())
    return fail(KV_ERR_STATE, "kv_seq_swap_in: unknown sequence %lld", (long long)seq);
  kv_pool::Seq& s = it->second;
  if (!s.swapped)
    return fail(KV_ERR_STATE, "kv_seq_swap_in: sequence %lld is not swapped out", (long long)seq);
  const int64_t need = ceil_div(s.len, p->cfg.block_size);
  *n = (int32_t)need;
  if (cap < need || (!ids_out && need > 0))
    return fail(KV_ERR_INVALID, "kv_seq_swap_in: capacity %d < %lld", cap, (long long)need);
  if (need > (int64_t)p->free_stack.size())
    return fail(KV_ERR_OOM, "kv_seq_swap_in: need %lld blocks, %zu free", (long long)need,
                p->free_stack.size());
  s.blocks.resize(need);
  for (int64_t i = 0; i < need; ++i) {
    const int32_t b = p->free_stack.back();
    p->free_stack.pop_back();
    p->refcount[b] = 1;
    s.blocks[i] = b;
    ids_out[i] = b;
  }
  s.swapped = false;
  return KV_OK;
}

int32_t kv_pool_shared_blocks(const kv_pool_t* p) {
  if (!p) return -1;
  int32_t n = 0;
  for (const int32_t r : p->refcount) n += r > 1 ? 1 : 0;
  return n;
}

// Blocks a step's sequences share, other than the prefix a shared-prefix
// step reads once, are read by several sequences in one launch: keep them in
// the caches.
kv_load_policy kv_paged_attention_choose_load_policy(const kv_pool_t* p, int32_t shared_tokens) {
  if (!p) return KV_LOADS_STREAM;
  const int32_t common = shared_tokens > 0 ? shared_tokens / p->cfg.block_size : 0;
  return kv_pool_shared_blocks(p) > common ? KV_LOADS_CACHED : KV_LOADS_STREAM;
}

int32_t kv_seq_is_swapped(const kv_pool_t* p, int64_t seq) {
  if (!p) return -1;
  auto it = p->seqs.find(seq);
  return it == p->seqs.end() ? -1 : (it->second.swapped ? 1 : 0);
}

const char* kv_last_error(void) { return pagedkv::g_last_error.c_str(); }

}  // extern "C"
