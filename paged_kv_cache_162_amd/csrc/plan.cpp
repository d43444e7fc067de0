// Host-side work plans for paged decode attention and chunked prefill.
//
// The decode kernel runs one workgroup per (sequence, KV head, context
// partition). Built from the host's copy of the context lengths, the plan
// lists exactly the (sequence, partition) pairs that hold tokens, so the grid
// has no idle workgroups, and one item per empty (or invalid) sequence so its
// output is still written.
//
// Placement. Every item becomes num_kv_heads consecutive workgroups, and the
// hardware deals workgroups out in order: workgroup w goes to XCD w % 8 and
// there, in turn, to its next compute unit, so on a device of N compute units
// w lands on slot w % N while the whole grid is resident (it is for decode
// batches: one wave per workgroup, several waves per CU). Each CU streams its
// waves' K/V through one memory pipeline, so the kernel ends when the most
// loaded CU has read its bytes (measured on MI355X: packing the longest
// partitions two, four or eight to a CU slows the 70B-shaped step from 65 to
// 72, 77 and 98 us). Items i and i + T with T = N / gcd(num_kv_heads, N) land
// on the same slots. The plan therefore sorts the items longest first and lays
// them out in rows, every other row reversed, so that each slot class gets
// long and short items alike and the per-CU loads even out: rows of 2T (two
// rounds of the device) when num_kv_heads divides N, so that a round holds
// whole items, and rows of T otherwise. Measured on MI355X, one box per
// comparison: 70B-shaped step (8 KV heads) 66.0 us against 68.8 us for
// longest first alone; then rows of 2T, 4T and 8T 64.9, 65.1 and 67.8 us
// against 65.1 us for rows of T (four runs each); 13B-shaped MHA step (40 KV
// heads) 261.7 us with rows of T against 270.4 us with rows of 2T. With no
// placement model (num_kv_heads or num_cus <= 0) the order is longest first.

#include <algorithm>
#include <cstdint>
#include <numeric>
#include <vector>

#include "../../include/pagedkv.h"
#include "status.h"

using pagedkv::fail;

extern "C" kv_status kv_paged_attention_plan(const int32_t* context_lens_host, int32_t S,
                                             int32_t partition_size, int32_t num_kv_heads,
                                             int32_t num_cus, int32_t* items_out, int32_t cap,
                                             int32_t* n_items) {
  pagedkv::clear_error();
  const int32_t P = partition_size == 0 ? 512 : partition_size;
  if (!n_items || S < 0 || (S > 0 && !context_lens_host))
    return fail(KV_ERR_INVALID, "kv_paged_attention_plan: null argument or negative S");
  if (P < 16 || P > 1024 || P % 16 != 0)
    return fail(KV_ERR_INVALID, "kv_paged_attention_plan: partition_size %d", partition_size);
  struct Item {
    int32_t s, p, len;
  };
  std::vector<Item> items;
  items.reserve((size_t)S * 2);
  for (int32_t s = 0; s < S; ++s) {
    const int32_t ctx = context_lens_host[s];
    if (ctx <= 0) {
      items.push_back({s, 0, -1});
      continue;
    }
    const int32_t np = (int32_t)(((int64_t)ctx + P - 1) / P);
    for (int32_t p = 0; p < np; ++p)
      items.push_back({s, p, std::min<int32_t>(P, ctx - p * P)});
  }
  std::stable_sort(items.begin(), items.end(),
                   [](const Item& a, const Item& b) { return a.len > b.len; });
  *n_items = (int32_t)items.size();
  if ((size_t)cap < items.size() || (!items_out && !items.empty()))
    return fail(KV_ERR_INVALID, "kv_paged_attention_plan: capacity %d < %zu items", cap,
                items.size());
  size_t period = items.size();  // no placement model: one row, longest first
  if (num_kv_heads > 0 && num_cus > 0)
    period = (size_t)(num_cus / std::gcd(num_kv_heads, num_cus)) *
             (num_cus % num_kv_heads == 0 ? 2 : 1);
  for (size_t row = 0; row * period < items.size(); ++row) {
    const size_t lo = row * period, hi = std::min(items.size(), lo + period);
    for (size_t i = lo; i < hi; ++i) {
      const Item& it = items[(row & 1) ? lo + (hi - 1 - i) : i];
      items_out[2 * i] = it.s;
      items_out[2 * i + 1] = it.p;
    }
  }
  return KV_OK;
}

// Plan for the chunked-prefill kernel, which runs one workgroup per
// (sequence, KV head, block of query rows): one item per block of
// kv_paged_attention_prefill_rows_per_item rows of each sequence's chunk,
// ordered by the number of keys the block's last row sees, most first, so
// the longest workgroups start first. Blocks of an impossible sequence (chunk
// longer than its context) come last; the kernel writes NaN for them.
extern "C" kv_status kv_paged_attention_prefill_plan(const int32_t* query_start_host,
                                                     const int32_t* context_lens_host, int32_t S,
                                                     int32_t num_q_heads, int32_t num_kv_heads,
                                                     int32_t* items_out, int32_t cap,
                                                     int32_t* n_items) {
  pagedkv::clear_error();
  if (!n_items || S < 0 || (S > 0 && (!query_start_host || !context_lens_host)))
    return fail(KV_ERR_INVALID, "kv_paged_attention_prefill_plan: null argument or negative S");
  const int32_t rpb = kv_paged_attention_prefill_rows_per_item(num_q_heads, num_kv_heads);
  if (rpb <= 0)
    return fail(KV_ERR_UNSUPPORTED, "kv_paged_attention_prefill_plan: heads %d / %d", num_q_heads,
                num_kv_heads);
  struct Item {
    int32_t s, b;
    int64_t keys;
  };
  std::vector<Item> items;
  for (int32_t s = 0; s < S; ++s) {
    const int64_t C = (int64_t)query_start_host[s + 1] - query_start_host[s];
    if (C <= 0) continue;
    const int64_t L = context_lens_host[s];
    const int64_t nb = (C + rpb - 1) / rpb;
    for (int64_t b = 0; b < nb; ++b) {
      const int64_t keys = L < C ? -1 : (L - C) + std::min<int64_t>((b + 1) * rpb, C);
      items.push_back({s, (int32_t)b, keys});
    }
  }
  std::stable_sort(items.begin(), items.end(),
                   [](const Item& a, const Item& b) { return a.keys > b.keys; });
  *n_items = (int32_t)items.size();
  if ((size_t)cap < items.size() || (!items_out && !items.empty()))
    return fail(KV_ERR_INVALID, "kv_paged_attention_prefill_plan: capacity %d < %zu items", cap,
                items.size());
  for (size_t i = 0; i < items.size(); ++i) {
    items_out[2 * i] = items[i].s;
    items_out[2 * i + 1] = items[i].b;
  }
  return KV_OK;
}

// Key runs for a prefill launch (kv_paged_attention_prefill_split): none
// while the plan's units cover min_units; else as many as reach it, each run
// keeping at least kPrefillMinRunTiles tiles of the longest item.
constexpr int64_t kPrefillMinRunTiles = 16;  // 512 keys

extern "C" int32_t kv_paged_attention_prefill_choose_splits(const int32_t* query_start_host,
                                                            const int32_t* context_lens_host,
                                                            int32_t S, int32_t num_q_heads,
                                                            int32_t num_kv_heads,
                                                            int32_t min_units) {
  const int32_t rpb = kv_paged_attention_prefill_rows_per_item(num_q_heads, num_kv_heads);
  if (rpb <= 0 || S <= 0 || !query_start_host || !context_lens_host || min_units <= 0) return 1;
  int64_t items = 0, max_tiles = 0;
  for (int32_t s = 0; s < S; ++s) {
    const int64_t C = (int64_t)query_start_host[s + 1] - query_start_host[s];
    const int64_t L = context_lens_host[s];
    if (C <= 0 || L < C) continue;
    items += (C + rpb - 1) / rpb;
    max_tiles = std::max<int64_t>(max_tiles, (L + 31) / 32);  // the last block sees every key
  }
  const int64_t units = items * num_kv_heads;
  if (units == 0 || units >= min_units) return 1;
  int64_t splits = (min_units + units - 1) / units;
  splits = std::min<int64_t>(splits, max_tiles / kPrefillMinRunTiles);
  splits = std::min<int64_t>(splits, KV_PREFILL_MAX_SPLITS);
  return (int32_t)std::max<int64_t>(1, splits);
}

// A partition size for a decode batch: the largest of 1024, 768 and 512
// tokens (a multiple of the block size) whose
// work units - KV heads times the partitions of every sequence - still
// number at least min_units, else 512. Longer partitions mean fewer units to
// start, fewer partial results and less merge work; min_units keeps enough
// units to cover the device (measured on MI355X: about 3/4 of the 2048
// waves it runs at once, 256 CUs x 8 waves).
extern "C" int32_t kv_paged_attention_choose_partition(const int32_t* context_lens_host,
                                                       int32_t S, int32_t num_kv_heads,
                                                       int32_t block_size, int32_t min_units) {
  if (S <= 0 || !context_lens_host || num_kv_heads <= 0 || block_size <= 0) return 512;
  for (const int32_t P : {1024, 768}) {
    if (P % block_size != 0) continue;
    int64_t units = 0;
    for (int32_t s = 0; s < S; ++s) {
      const int64_t ctx = context_lens_host[s];
      units += ctx > 0 ? (ctx + P - 1) / P : 1;
    }
    if (units * num_kv_heads >= min_units) return P;
  }
  return 512;
}

// ---- step policies --------------------------------------------------------
// How many leading positions a decode batch shares, and whether the
// shared-prefix step should read them once for the batch. The thresholds are
// measurements on MI355X, stated in the header. (The load-policy choice needs
// the pool's reference counts and sits with the block manager.)

namespace {
constexpr int32_t kSharedMinSeqs = 4;
constexpr int32_t kSharedMinTokens = 256;
constexpr int64_t kSharedMinReads = 49152;  // sequences x shared positions
// an fp8 cache saves half the bytes per position read once instead of per
// sequence, so the prefix must be read about twice as often to pay
constexpr int64_t kSharedMinReadsFp8 = 98304;
}  // namespace

extern "C" int32_t kv_paged_attention_common_prefix(const int32_t* tables_host, int32_t S,
                                                    int32_t max_blocks,
                                                    const int32_t* context_lens_host,
                                                    int32_t block_size) {
  if (S <= 0 || !tables_host || !context_lens_host || max_blocks <= 0 || block_size <= 0)
    return 0;
  int64_t min_len = context_lens_host[0];
  for (int32_t s = 1; s < S; ++s) min_len = std::min<int64_t>(min_len, context_lens_host[s]);
  // blocks wholly before every sequence's last position, within the table
  const int64_t kmax = std::min<int64_t>(min_len - 1, (int64_t)max_blocks * block_size) / block_size;
  int64_t k = 0;
  for (; k < kmax; ++k) {
    const int32_t id = tables_host[k];
    bool same = true;
    for (int32_t s = 1; s < S && same; ++s) same = tables_host[(size_t)s * max_blocks + k] == id;
    if (!same) break;
  }
  return (int32_t)(k * block_size);
}

extern "C" int32_t kv_paged_attention_choose_shared_prefix(
    const int32_t* tables_host, int32_t S, int32_t max_blocks, const int32_t* context_lens_host,
    int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    kv_dtype dtype) {
  if ((dtype != KV_F16 && dtype != KV_BF16 && dtype != KV_FP8_E4M3) || head_dim != 128 ||
      num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || num_q_heads / num_kv_heads > 16 ||
      S < kSharedMinSeqs)
    return 0;
  int32_t shared =
      kv_paged_attention_common_prefix(tables_host, S, max_blocks, context_lens_host, block_size);
  if (shared > KV_SHARED_PREFIX_MAX_TOKENS)  // whole blocks: every block size divides the limit
    shared = KV_SHARED_PREFIX_MAX_TOKENS;
  const int64_t min_reads = dtype == KV_FP8_E4M3 ? kSharedMinReadsFp8 : kSharedMinReads;
  return (shared < kSharedMinTokens || (int64_t)S * shared < min_reads) ? 0 : shared;
}
