/*
 * pagedkv - paged KV cache and paged decode attention for AMD Instinct MI355X
 * (gfx950). C ABI of libpagedkv.so.
 *
 * Pages cited in this header:
 *   [1] "PagedAttention - how vLLM stopped wasting 80% of your GPU memory"
 *       (shivam2003.com/posts/pagedattention.html)
 *   [2] "PagedAttention: How vLLM Borrowed Virtual Memory to Unlock GPU
 *       Serving at Scale" (fp4-site.pages.dev/system/pagedattention-vllm-deep-dive/)
 *   [3] "PagedAttention and vLLM: Virtual Memory for the KV Cache"
 *       (passgenai.com, NCA-GENL course lesson 12-07)
 *   [4] "What is paged attention?" (netraruntime.com/learn/paged-attention)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every call returns kv_status (or a plain value where stated). On an error
 *   kv_last_error() returns a message for the calling thread.
 * - Host operations on a pool are all-or-nothing: on any error no block,
 *   reference count, table or length changes ([3], "L3": preemption and
 *   admission are all-or-nothing per sequence).
 * - A kv_pool_t is host metadata only. It is not thread-safe: callers
 *   serialise calls on one handle.
 * - Device entry points take device pointers owned by the caller (PyTorch in
 *   the bundled binding) and a hipStream_t. The library never allocates or
 *   frees device memory and never synchronises; work is enqueued on the
 *   given stream. Argument checks happen on the host before any launch; a
 *   failed launch returns KV_ERR_HIP.
 * - Cache layout, per layer ([2], "The Custom CUDA Kernel"): a K pool and a V
 *   pool, each [num_blocks][num_kv_heads][block_size][head_dim], row-major,
 *   elements of one kv_dtype; the leading index is the physical block ID.
 * - Token position p of a sequence lives in slot
 *   table[p / B] * B + p % B ([4], "How it works"); slot s is element
 *   [s / B][h][s % B][:] of a pool.
 * - Supported by the decode kernels: block_size 8, 16 or 32 (16 is the
 *   pages' default; [1] "Why 16 tokens per block specifically?" treats it as
 *   a tuning knob), head_dim 64 or 128, num_q_heads a multiple of
 *   num_kv_heads, dtypes f32/f16/bf16. Anything else returns
 *   KV_ERR_UNSUPPORTED. Slot mapping, cache writes and block copies take any
 *   block size.
 */
#ifndef PAGEDKV_H_
#define PAGEDKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

typedef enum {
  KV_OK = 0,
  KV_ERR_INVALID = -1,     /* bad argument (null pointer, size, out-of-range ID) */
  KV_ERR_OOM = -2,         /* not enough free blocks; nothing changed */
  KV_ERR_UNSUPPORTED = -3, /* shape or dtype the device kernels do not cover */
  KV_ERR_HIP = -4,         /* the HIP runtime reported an error at launch */
  KV_ERR_STATE = -5        /* wrong object state: unknown sequence, block not held */
} kv_status;

/* KV_FP8_E4M3: one byte per element, the OCP E4M3 float (sign, 4 exponent
 * bits with bias 7, 3 mantissa bits, no infinities, 0x7F/0xFF NaN, largest
 * magnitude 448). It describes a pool's storage only (kv_pool_create,
 * kv_quantize_fp8 output); the _fp8 device entry points below read and write
 * such pools, with the query / new-token type given separately. */
typedef enum { KV_F32 = 0, KV_F16 = 1, KV_BF16 = 2, KV_FP8_E4M3 = 3 } kv_dtype;

typedef struct {
  int32_t num_blocks;   /* physical blocks in the pool, > 0 */
  int32_t block_size;   /* tokens per block, > 0 (the device path needs 16) */
  int32_t num_layers;   /* layers sharing one block ID space, > 0 */
  int32_t num_kv_heads; /* > 0 */
  int32_t head_dim;     /* > 0 */
  kv_dtype dtype;
} kv_pool_config;

typedef struct kv_pool kv_pool_t; /* opaque; host metadata only */

/* ---------------------------------------------------------------------------
 * Host: block pool ([3], "L2 - Mechanism", the block pool; [4], "How it
 * works": allocation pops the free list and freeing pushes it, both O(1)).
 * ------------------------------------------------------------------------- */

/* Create the host metadata for a pool of uniform blocks, all free. The
 * initial free order hands out block 0 first, then 1, 2, ... ([1], "A small
 * worked example": the first free blocks are P0 and P1). *out receives the
 * handle; release it with kv_pool_destroy. */
kv_status kv_pool_create(const kv_pool_config* cfg, kv_pool_t** out);
void kv_pool_destroy(kv_pool_t* pool);

/* Replace the free order: afterwards blocks are handed out as order[0],
 * order[1], ... `order` must be a permutation of [0, num_blocks) (n ==
 * num_blocks). Only allowed while every block is free (KV_ERR_STATE
 * otherwise). Used to place sequences in shuffled physical blocks. */
kv_status kv_pool_set_free_order(kv_pool_t* pool, int32_t n, const int32_t* order);

/* Bytes of ONE layer's K pool (equal to its V pool):
 * num_blocks * num_kv_heads * block_size * head_dim * element size. */
size_t kv_pool_layer_bytes(const kv_pool_t* pool);
/* Resident-token capacity num_blocks * block_size ([3], "L2": the block
 * count is the hard capacity, however tokens are spread). -1 on NULL. */
int64_t kv_pool_capacity_tokens(const kv_pool_t* pool);
int32_t kv_num_free_blocks(const kv_pool_t* pool);

/* Pop n blocks (reference count 1 each) into ids_out[0..n). All or nothing:
 * KV_ERR_OOM if fewer than n are free. */
kv_status kv_block_alloc(kv_pool_t* pool, int32_t n, int32_t* ids_out);
/* Add one reference per listed block ([1], "Memory sharing": a reference
 * count per physical block). Every block must be held (KV_ERR_STATE). */
kv_status kv_block_incref(kv_pool_t* pool, int32_t n, const int32_t* ids);
/* Drop one reference per listed block; blocks reaching zero are pushed on the
 * free list in reverse list order, so the next allocations return them in
 * list order. KV_ERR_STATE if a block would drop below zero. */
kv_status kv_block_free(kv_pool_t* pool, int32_t n, const int32_t* ids);
/* Current reference count, 0 if free, -1 for an ID outside the pool. */
int32_t kv_block_refcount(const kv_pool_t* pool, int32_t id);

/* ---------------------------------------------------------------------------
 * Host: sequences ([3], "The allocation lifecycle"; [2], "Walking Through the
 * Lifecycle"; copy-on-write per [2], "Copy-on-Write for Beam Search and
 * Parallel Sampling").
 * ------------------------------------------------------------------------- */

/* New empty sequence; handles are never reused within a pool. */
kv_status kv_seq_create(kv_pool_t* pool, int64_t* seq_out);
/* New sequence sharing every block of `parent` (each gains a reference). */
kv_status kv_seq_fork(kv_pool_t* pool, int64_t parent, int64_t* child_out);
/* Reserve n_tokens new positions at the end of `seq`.
 * - Growth is lazy: a block is taken just before position p with
 *   p % block_size == 0, so t tokens hold ceil(t / block_size) blocks
 *   ([4], "How it works").
 * - If the first new position falls inside the last block and that block's
 *   reference count exceeds one, the block is copied: a new block is taken,
 *   the old one loses a reference, the table entry is redirected, and the
 *   pair is reported in (cow_src[0], cow_dst[0]) with *n_cow = 1. The caller
 *   must run kv_copy_blocks on that pair before writing the new tokens.
 *   Otherwise *n_cow = 0. Appending after a full shared block copies nothing
 *   ([1], "A small worked example", step 3).
 * - slots_out[i] receives the slot of position len + i (int64).
 * - The copy block (if any) is taken before the new blocks.
 * All or nothing (KV_ERR_OOM). slots_out may be NULL when n_tokens == 0;
 * cow_src, cow_dst and n_cow must not be NULL. */
kv_status kv_seq_append(kv_pool_t* pool, int64_t seq, int32_t n_tokens, int64_t* slots_out,
                        int32_t* cow_src, int32_t* cow_dst, int32_t* n_cow);
/* Return every block of the sequence ([2], "Sequence Completion"): one
 * reference each, pushed in reverse logical order when it reaches zero. */
kv_status kv_seq_free(kv_pool_t* pool, int64_t seq);
/* Copy the block table into ids[0..*n). If cap < the table length, returns
 * KV_ERR_INVALID with *n set to the length needed. */
kv_status kv_seq_block_table(const kv_pool_t* pool, int64_t seq, int32_t cap, int32_t* ids,
                             int32_t* n);
/* Tokens held by the sequence, -1 if the handle is unknown. */
int32_t kv_seq_len(const kv_pool_t* pool, int64_t seq);
/* Pack the tables of n_seqs sequences into a row-major host array
 * tables_out[n_seqs][max_blocks] (unused entries = -1) and their lengths into
 * lens_out[n_seqs]. KV_ERR_INVALID if a table is wider than max_blocks. */
kv_status kv_seq_pack_tables(const kv_pool_t* pool, int32_t n_seqs, const int64_t* seqs,
                             int32_t max_blocks, int32_t* tables_out, int32_t* lens_out);

/* Swap a sequence out under memory pressure ([3], "The allocation
 * lifecycle": preempt a sequence by moving its blocks to host memory; [1],
 * "Preemption"): ids[0..*n) receive the sequence's current table (the blocks
 * whose contents the caller copies to the host, e.g. with kv_swap_out_blocks,
 * before any later write can reuse them), then each block loses one
 * reference exactly as kv_seq_free does. The sequence keeps its length and
 * is marked swapped out. If cap < the table length, returns KV_ERR_INVALID
 * with *n set and nothing changed. KV_ERR_STATE if unknown or already
 * swapped out. A swapped-out sequence cannot be appended to, forked, or
 * packed / read by kv_seq_block_table (KV_ERR_STATE); it can be freed. */
kv_status kv_seq_swap_out(kv_pool_t* pool, int64_t seq, int32_t cap, int32_t* ids, int32_t* n);
/* Readmit a swapped-out sequence: takes ceil(len / block_size) free blocks
 * (reference count 1, all or nothing: KV_ERR_OOM changes nothing) and
 * returns them in logical order in ids[0..*n); the caller copies the saved
 * contents into them (kv_swap_in_blocks). Blocks that were shared before
 * the swap come back as private copies. KV_ERR_STATE if the sequence is
 * unknown or not swapped out; KV_ERR_INVALID with *n set if cap is short. */
kv_status kv_seq_swap_in(kv_pool_t* pool, int64_t seq, int32_t cap, int32_t* ids, int32_t* n);
/* 1 if the sequence is swapped out, 0 if resident, -1 if unknown. */
int32_t kv_seq_is_swapped(const kv_pool_t* pool, int64_t seq);
/* Number of blocks currently held by more than one reference (shared by
 * forks or prefixes, [1] "Memory sharing"); -1 for a null pool. */
int32_t kv_pool_shared_blocks(const kv_pool_t* pool);

/* ---------------------------------------------------------------------------
 * Device: slot mapping and cache writes.
 * ------------------------------------------------------------------------- */

/* slots[i] = tables[seq_idx[i]][pos[i] / block_size] * block_size
 *            + pos[i] % block_size, as int64 ([4], "How it works").
 * Entries that cannot be mapped (seq_idx outside [0, num_rows), pos < 0,
 * pos / block_size >= max_blocks, a negative table entry) give -1, which
 * kv_reshape_and_cache skips. tables is [num_rows][max_blocks] int32; seq_idx
 * and pos are int32 [n]; slots is int64 [n]; all device pointers. */
kv_status kv_slot_mapping(const int32_t* tables, int32_t num_rows, int32_t max_blocks,
                          const int32_t* seq_idx, const int32_t* pos, int32_t n,
                          int32_t block_size, int64_t* slots, hipStream_t stream);

/* Write each new token's K and V into its slot ([3], "The allocation
 * lifecycle": each decode step writes the token's K,V into the last block).
 * k_new, v_new: [n][num_kv_heads][head_dim] of `dtype`; k_pool, v_pool: one
 * layer's pools with num_blocks blocks; slots: int64 [n]. The copy is bit
 * exact. Slots < 0 or >= num_blocks * block_size are skipped. Slots must be
 * distinct within a call (duplicates race). Pointers must be 16-byte
 * aligned. */
kv_status kv_reshape_and_cache(const void* k_new, const void* v_new, void* k_pool,
                               void* v_pool, const int64_t* slots, int32_t n,
                               int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, kv_dtype dtype, hipStream_t stream);

/* Slot mapping and cache write of a batch of new tokens in one launch: token
 * i (i < n) goes to position pos[i] of sequence seq_idx[i]; its slot is
 * computed as kv_slot_mapping does ([4], "How it works"), stored in slots[i],
 * and its K and V rows are copied there as kv_reshape_and_cache does ([3],
 * "The allocation lifecycle": each decode step writes the new token's K,V
 * into the last block). Arguments as for those two calls: tables
 * [num_rows][max_blocks] int32, seq_idx and pos int32 [n], k_new and v_new
 * [n][num_kv_heads][head_dim] of `dtype`, slots int64 [n]; all device
 * pointers. Unmappable tokens get slot -1 and are not written. The copy is
 * bit exact; slots must be distinct within a call. */
kv_status kv_append_tokens(const int32_t* tables, int32_t num_rows, int32_t max_blocks,
                           const int32_t* seq_idx, const int32_t* pos, int32_t n,
                           const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                           int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, kv_dtype dtype, int64_t* slots,
                           hipStream_t stream);

/* Device half of copy-on-write ([2], "Copy-on-Write ...": copy the shared
 * block's content into the new block): for every pair (pairs[2i] = src,
 * pairs[2i+1] = dst) and every layer, copy block_bytes bytes of K and of V
 * from block src to block dst. k_pools and v_pools are HOST arrays of
 * num_layers device pointers (num_layers <= 256); pairs is a device int32
 * array of 2n entries; every src and dst must be < num_blocks (checked on
 * the device: out-of-range pairs are skipped). block_bytes must be a
 * multiple of 16 and the pools 16-byte aligned. Pairs must not chain (a dst
 * that is also a src in the same call). */
kv_status kv_copy_blocks(void* const* k_pools, void* const* v_pools, int32_t num_layers,
                         const int32_t* pairs, int32_t n, int32_t num_blocks,
                         size_t block_bytes, hipStream_t stream);

/* Device half of a swap ([3], "The allocation lifecycle", memory
 * pressure): copy whole blocks - every layer, K and V - between the pools and
 * host memory. block_ids is a device int32 array of n physical IDs (entries
 * outside [0, num_blocks) are skipped); k_pools and v_pools are HOST arrays
 * of num_layers (<= 256) device pointers; block_bytes is one layer's bytes
 * of one block in one pool (num_kv_heads * block_size * head_dim * element
 * size, a multiple of 16). host_buffer must be pinned host memory
 * (hipHostMalloc, torch pin_memory) of n * num_layers * 2 * block_bytes bytes,
 * laid out [n][num_layers][K, V][block_bytes]; the kernel reads or writes it
 * directly, so it must stay allocated until the stream has passed the copy.
 * The copy is bit exact. KV_ERR_INVALID for unpinned or misaligned buffers. */
kv_status kv_swap_out_blocks(void* const* k_pools, void* const* v_pools, int32_t num_layers,
                             const int32_t* block_ids, int32_t n, int32_t num_blocks,
                             size_t block_bytes, void* host_buffer, hipStream_t stream);
kv_status kv_swap_in_blocks(void* const* k_pools, void* const* v_pools, int32_t num_layers,
                            const int32_t* block_ids, int32_t n, int32_t num_blocks,
                            size_t block_bytes, const void* host_buffer, hipStream_t stream);

/* Measurement utility, not a step of the method: reads `bytes` (a multiple of
 * 16) of device memory at src (16-byte aligned) with the decode kernels'
 * non-temporal 16-byte loads, `workgroups` workgroups of 256 threads striding
 * over the buffer, and writes one checksum word per workgroup to sink (device
 * uint32 [workgroups]). Its bytes per second over a buffer far larger than
 * the last-level cache are the HBM read rate a streaming kernel reaches on the
 * device, the ceiling beside the published peak. */
kv_status kv_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                            hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Device: paged decode attention ([1], "The PagedAttention kernel"; [2],
 * "The Custom CUDA Kernel"; [3], "The kernel change").
 * ------------------------------------------------------------------------- */

/* Work plan for kv_paged_attention_decode, built on the host from the host
 * copy of the context lengths (the block manager has them): the list of
 * (sequence, partition) items that hold tokens, and one item for each
 * sequence of length <= 0 (so its output is still written), every item once.
 * Order: longest first, laid out for the device's workgroup placement.
 * Item i becomes workgroups i*num_kv_heads .. i*num_kv_heads + num_kv_heads - 1,
 * which the hardware deals to compute units in turn, so items i and i + T,
 * T = num_cus / gcd(num_kv_heads, num_cus), share compute units; the sorted
 * items go out in rows with every other row reversed, which evens out the
 * K/V bytes each compute unit streams: rows of 2T when num_kv_heads divides
 * num_cus, of T otherwise (the lengths that measured fastest). num_kv_heads or num_cus <= 0:
 * plain longest-first order. num_cus is the device's compute-unit count
 * (hipDeviceAttributeMultiprocessorCount, 256 on MI355X).
 * items_out: host int32 [cap][2] receiving (sequence, partition) pairs;
 * *n_items receives the item count, which is at most
 * S * ceil(max_len / partition) (KV_ERR_INVALID with *n_items set if cap is
 * smaller). partition_size as for the decode (0 = 512). The caller copies
 * the items to the device and passes them to the decode with the same
 * lengths, partition size and KV head count. */
kv_status kv_paged_attention_plan(const int32_t* context_lens_host, int32_t S,
                                  int32_t partition_size, int32_t num_kv_heads, int32_t num_cus,
                                  int32_t* items_out, int32_t cap, int32_t* n_items);

/* Workspace bytes kv_paged_attention_decode needs for these sizes: 0 when
 * max_context_len <= the partition size (every sequence finishes in one
 * partition), else S * num_q_heads * num_partitions * (head_dim + 2) * 4.
 * Layout (fp32): partial outputs [S][num_kv_heads][num_partitions][G][head_dim]
 * then partial (max, sum) pairs [S][num_kv_heads][num_partitions][G][2],
 * G = num_q_heads / num_kv_heads, so one work unit's partials are
 * contiguous. partition_size 0 picks the default (512). Returns 0 for
 * invalid sizes. The workspace needs no initialisation; calls that run
 * concurrently need separate workspaces. */
size_t kv_paged_attention_workspace_bytes(int32_t S, int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t max_context_len,
                                          int32_t partition_size);

/* How the decode kernels load K and V (the load_policy argument of every
 * decode entry point):
 *   KV_LOADS_STREAM  loads carry the non-temporal hint: every block is read
 *                    once per step, so nothing is kept in the caches for it.
 *                    Fastest when no block is shared between the step's
 *                    sequences (measured 10-15% over plain loads).
 *   KV_LOADS_CACHED  plain loads: blocks shared by several sequences (a
 *                    common prefix, [1] "Memory sharing") stay in the caches
 *                    for their next reader.
 * Results are identical under both; kv_paged_attention_choose_load_policy
 * picks one for a step from the pool's sharing. Any other value is
 * KV_ERR_INVALID. */
typedef enum { KV_LOADS_STREAM = 0, KV_LOADS_CACHED = 1 } kv_load_policy;

/* out[s][hq][:] = sum_j softmax_j(scale * <q[s][hq], K_s[j]>) V_s[j] over the
 * first context_lens[s] positions of sequence s, where K_s[j] and V_s[j] are
 * read from slot(j) of KV head hq / (num_q_heads / num_kv_heads) - exactly
 * the attention of the contiguous cache ([1], "The PagedAttention kernel").
 *
 * out:          device float [S][num_q_heads][head_dim] (fp32 output)
 * q:            device [S][num_q_heads][head_dim] of `dtype`
 * k_pool/v_pool device, one layer's pools with num_blocks blocks
 * block_tables: device int32 [S][max_blocks]
 * context_lens: device int32 [S]
 * max_context_len: host upper bound on every context_lens[s]; it sizes the
 *               grid (number of partitions).
 * partition_size: tokens per work item: a multiple of 16 and of block_size,
 *               at most 1024 tokens; 0 = 512.
 *               Sequences longer than one partition are split and a second
 *               kernel merges the partial results with a log-sum-exp
 *               reduction ([2], "The Custom CUDA Kernel": per-piece partial
 *               outputs and denominators merged stably), in partition
 *               order, so results do not depend on scheduling.
 * work_items:   optional device int32 [n_items][2] from
 *               kv_paged_attention_plan; the grid is then exactly n_items *
 *               num_kv_heads workgroups. NULL: the grid covers every possible
 *               partition, S * num_kv_heads * ceil(max_context_len /
 *               partition), and workgroups past a sequence's end exit at once.
 *               Items whose sequence or partition is out of range are skipped.
 * workspace:    device scratch of at least
 *               kv_paged_attention_workspace_bytes(...) bytes (may be NULL
 *               when that is 0).
 * load_policy:  how K and V are loaded (kv_load_policy above).
 *
 * Per-sequence device-side checks (no fault, no error code): a sequence with
 * context_lens[s] == 0 gets an all-zero output. A sequence whose length is
 * negative, exceeds max_blocks * block_size or max_context_len, or whose
 * live table entries fall outside [0, num_blocks), gets NaN in every output
 * element, and no out-of-range memory is read.
 *
 * Kernels: head groups of 2..16 query heads per KV head with f16/bf16 and
 * head_dim 128 run on MFMA matrix cores; other cases run on the vector ALUs.
 * One workgroup (a single wave64) handles one (sequence, KV head,
 * partition). A call is one kernel launch, plus the merge launch when
 * max_context_len exceeds the partition size. */
kv_status kv_paged_attention_decode(float* out, const void* q, const void* k_pool,
                                    const void* v_pool, const int32_t* block_tables,
                                    int32_t max_blocks, const int32_t* context_lens, int32_t S,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t num_blocks, float scale,
                                    kv_dtype dtype, int32_t partition_size,
                                    int32_t max_context_len, const int32_t* work_items,
                                    int32_t n_items, void* workspace, size_t ws_bytes,
                                    kv_load_policy load_policy, hipStream_t stream);

/* A partition size for a decode batch, from the host copy of its context
 * lengths: the largest of 1024, 768 and 512 tokens that is a multiple of
 * block_size and still gives at least min_units work units (num_kv_heads x
 * the partitions of every sequence), else 512. Fewer, longer units start
 * less work, write fewer partials and leave less to merge; min_units keeps
 * the device covered (about 1500 measured best on MI355X: 3/4 of 256 CUs x
 * 8 waves). Returns 512 for empty or invalid input. */
int32_t kv_paged_attention_choose_partition(const int32_t* context_lens_host, int32_t S,
                                            int32_t num_kv_heads, int32_t block_size,
                                            int32_t min_units);

/* Positions that all S sequences reach through the same leading table
 * entries, i.e. the same physical blocks ([1] "Memory sharing"), counted in
 * whole blocks and short of every sequence's last position (the block that
 * takes the step's new token never counts): k * block_size for the largest k
 * with tables[s][i] == tables[0][i] for every s and i < k and
 * k * block_size < context_lens[s] for every s. Host arrays: tables
 * [S][max_blocks] int32, context_lens [S]. 0 for S == 0 or invalid sizes. */
int32_t kv_paged_attention_common_prefix(const int32_t* tables_host, int32_t S,
                                         int32_t max_blocks, const int32_t* context_lens_host,
                                         int32_t block_size);

/* Shared positions for kv_paged_attention_decode_append_shared (dtype f16
 * or bf16: the pools' type) or kv_paged_attention_decode_append_shared_fp8
 * (dtype KV_FP8_E4M3: an fp8 cache), or 0 when a decode step over these
 * sequences should take the plain step: the common prefix above, where those
 * entry points support the step (head_dim 128, group size at most 16; a
 * common prefix longer than KV_SHARED_PREFIX_MAX_TOKENS is cut to it, the
 * rest left to the tails) and reading the prefix once per batch is expected
 * to be faster than once per sequence. The rule comes from shared/plain step
 * times measured on MI355X (32 query / 8 KV heads, bf16 queries, 4-128
 * sequences, 256-4096 shared positions, tails of 64 and 512 positions; a
 * point counts as faster at a time ratio of 0.97 or less): at least 4
 * sequences and 256 shared positions, and sequences x shared positions >=
 * 49,152 (16-bit cache) or >= 98,304 (fp8 cache, half the bytes saved per
 * read). 16-bit: every measured point with 65,536 prefix reads or more was
 * faster (ratios 0.34-0.89, whatever the tail), and of those with 32,768 or
 * fewer one was (0.88). fp8: every point with 131,072 reads or more was
 * faster (0.42-0.94), 3 of the 8 at 65,536, none below. Each threshold sits
 * between. */
int32_t kv_paged_attention_choose_shared_prefix(const int32_t* tables_host, int32_t S,
                                                int32_t max_blocks,
                                                const int32_t* context_lens_host,
                                                int32_t block_size, int32_t num_q_heads,
                                                int32_t num_kv_heads, int32_t head_dim,
                                                kv_dtype dtype);

/* Load policy for a decode step over pool: KV_LOADS_CACHED when the pool
 * holds shared blocks besides the shared_tokens / block_size prefix blocks
 * a shared-prefix step reads once by itself (those others are read by
 * several of the step's sequences and should stay in the caches), else
 * KV_LOADS_STREAM. shared_tokens 0 for a plain step. A null pool gives
 * KV_LOADS_STREAM. */
kv_load_policy kv_paged_attention_choose_load_policy(const kv_pool_t* pool,
                                                     int32_t shared_tokens);

/* One decode step with the cache write fused into the decode launch: for
 * each sequence s with t = context_lens[s] >= 1, position t-1 holds the
 * step's new token. Its K and V rows, k_new[s] and v_new[s]
 * ([S][num_kv_heads][head_dim] of `dtype`, device), are written to slot
 * block_tables[s][(t-1)/16]*16 + (t-1)%16 ([4], "How it works"; [3], "The
 * allocation lifecycle": each decode step writes the new token's K,V into
 * the last block), the slot is stored in slots[s] (device int64 [S]; -1
 * when t <= 0, the sequence is invalid or a table entry is out of range, in
 * which case nothing is written), and attention then runs exactly as
 * kv_paged_attention_decode over positions 0..t-1, the new token included.
 * On valid inputs, outputs, pools and slots are bit-identical to kv_slot_mapping +
 * kv_reshape_and_cache + kv_paged_attention_decode on the same inputs. The
 * block holding position t-1 must belong to s alone (run any copy-on-write
 * copy first). Other arguments, checks and launches as for
 * kv_paged_attention_decode; k_new and v_new must be 16-byte aligned. */
kv_status kv_paged_attention_decode_append(
    float* out, const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
    const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t S,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, float scale, kv_dtype dtype, int32_t partition_size,
    int32_t max_context_len, const int32_t* work_items, int32_t n_items, void* workspace,
    size_t ws_bytes, int64_t* slots, kv_load_policy load_policy, hipStream_t stream);

/* Bytes of the library's own split-K buffer used by
 * kv_paged_attention_decode_append_noalloc, on each GPU: 32 MiB. */
#define KV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* kv_paged_attention_decode_append without a workspace argument, for callers
 * that cannot allocate device memory: code under stream or graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. The split-K partials
 * go to a device buffer of KV_NOALLOC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on, from the first call there until the process ends
 * (the call looks up its address once per device; it calls no hipMalloc,
 * hipFree or other allocating routine). Arguments, checks, launches and
 * results are those of kv_paged_attention_decode_append: bit-identical
 * outputs, pools and slots for the same inputs. Sizes whose workspace
 * (kv_paged_attention_workspace_bytes) exceeds KV_NOALLOC_SCRATCH_BYTES get
 * KV_ERR_INVALID before anything is launched; e.g. 128 sequences x 64 query
 * heads with 768-token partitions fit contexts up to 5,376 tokens. Every call
 * on one GPU shares that GPU's buffer: calls that may overlap on one GPU
 * (different streams, no ordering between them) race and must not be made;
 * calls in one stream are ordered. The buffer needs no clearing between
 * calls (each call writes every partial it reads). */
kv_status kv_paged_attention_decode_append_noalloc(
    float* out, const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
    const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t S,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, float scale, kv_dtype dtype, int32_t partition_size,
    int32_t max_context_len, const int32_t* work_items, int32_t n_items, int64_t* slots,
    kv_load_policy load_policy, hipStream_t stream);

/* The decode step of kv_paged_attention_decode_append for a batch whose
 * sequences all share their first shared_tokens positions ([1] "Memory
 * sharing": the same physical blocks, reached through the same first
 * shared_tokens / block_size table entries). Attention over the shared
 * positions is computed once for all S queries - the shared blocks are read
 * once, not once per sequence - by a kernel whose workgroups each take 16
 * (sequence, query head) columns of one KV head and one range of the shared
 * positions, split into slices of at least 64 over up to 8 waves and merged
 * in LDS, so each range leaves one partial result per column; attention over
 * each sequence's own positions shared_tokens..t-1 runs in the decode kernels,
 * with the new token written as in kv_paged_attention_decode_append; the
 * prefix pass runs first, and the kernel that writes each tail's output (the
 * decode kernel, or the split-K merge for a tail spanning several
 * partitions) combines it with the prefix ranges through their softmax
 * denominators into the attention over positions 0..t-1 (the same value as
 * kv_paged_attention_decode_append, up to rounding order). Two launches
 * (three when a tail spans several partitions).
 *
 * shared_tokens: > 0, a multiple of block_size, at most
 *               KV_SHARED_PREFIX_MAX_TOKENS (KV_ERR_UNSUPPORTED beyond);
 *               the shared blocks are read through row 0 of block_tables.
 *               A sequence normally has
 *               context_lens[s] >= shared_tokens + 1 (its tail holds at
 *               least the new token); one of exactly shared_tokens gets the
 *               attention over the shared positions and no write (slots[s]
 *               = -1); a shorter one gets NaN.
 * max_tail_len: host bound on context_lens[s] - shared_tokens; it sizes
 *               the tail grid and the workspace (kv_paged_attention_
 *               workspace_bytes with max_context_len = max_tail_len).
 * work_items:   optional plan from kv_paged_attention_plan over the tail
 *               lengths context_lens[s] - shared_tokens.
 * aux:          device scratch of kv_paged_attention_shared_aux_bytes(S,
 *               num_q_heads, num_kv_heads, head_dim, shared_tokens) bytes,
 *               16-byte aligned: each prefix range's outputs and softmax
 *               denominators. Needs no initialisation; 0 from the size
 *               function means invalid sizes.
 * dtype f16 or bf16, head_dim 128, group size at most 16 (KV_ERR_UNSUPPORTED
 * otherwise); other arguments and checks as for
 * kv_paged_attention_decode_append. */
#define KV_SHARED_PREFIX_MAX_TOKENS 131072 /* 16 ranges x 8 slices x 1,024 */
size_t kv_paged_attention_shared_aux_bytes(int32_t S, int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t shared_tokens);
kv_status kv_paged_attention_decode_append_shared(
    float* out, const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
    const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t S,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, float scale, kv_dtype dtype, int32_t partition_size,
    int32_t shared_tokens, int32_t max_tail_len, const int32_t* work_items, int32_t n_items,
    void* workspace, size_t ws_bytes, float* aux, size_t aux_bytes, int64_t* slots,
    kv_load_policy load_policy, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * fp8 KV cache ([1], "How does this relate to quantization?": K and V stored
 * in 8 bits instead of 16 halve the bytes per element and compose with
 * paging; [3], the bytes_per_element term of the KV-size formula).
 *
 * Scheme (the pages fix none): the pools hold KV_FP8_E4M3 codes, laid out as
 * the 16-bit pools ([num_blocks][num_kv_heads][block_size][head_dim], one
 * byte per element). Each pool has one fp32 scale: a stored code c stands for
 * value(c) * scale. Writing x (f16 or bf16) stores the E4M3 code of
 * fp32(x / scale) - the fp32 quotient rounded to nearest even, then rounded
 * to the nearest E4M3 value with ties to the even code; magnitudes beyond 448
 * (and infinities) saturate to +-448, NaN is stored as 0x7F. Scales must be
 * finite and > 0 (else KV_ERR_INVALID).
 * ------------------------------------------------------------------------- */

/* As kv_reshape_and_cache, but k_new / v_new ([n][num_kv_heads][head_dim]
 * of `dtype`, f16 or bf16) are stored quantised with k_scale / v_scale into
 * fp8 pools. head_dim must be a multiple of 16; pools 8-byte aligned. */
kv_status kv_reshape_and_cache_fp8(const void* k_new, const void* v_new, void* k_pool,
                                   void* v_pool, const int64_t* slots, int32_t n,
                                   int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, kv_dtype dtype, float k_scale,
                                   float v_scale, hipStream_t stream);

/* dst[i] = E4M3 code of src[i] / scale for n elements (a multiple of 8) of
 * `dtype` (f16 or bf16); device pointers, src 16-byte and dst 8-byte
 * aligned. The same rounding as the cache writes; e.g. to convert a 16-bit
 * cache into an fp8 one. */
kv_status kv_quantize_fp8(const void* src, void* dst, int64_t n, kv_dtype dtype, float scale,
                          hipStream_t stream);

/* kv_paged_attention_decode over fp8 pools: the attention of the cache
 * values value(code) * k_scale (K) and value(code) * v_scale (V), i.e. the
 * same definition on the dequantised cache. q is [S][num_q_heads][head_dim]
 * of `dtype` (f16 or bf16); head_dim 64 or 128; group sizes 1..16; block
 * sizes 8, 16, 32. Each code is widened exactly to the query's type; at
 * head_dim 128 the MFMA path runs as for 16-bit pools, at head_dim 64 the
 * vector-ALU path. k_scale is folded into the score scale and v_scale into
 * the output. Other arguments, checks and workspace as for
 * kv_paged_attention_decode. */
kv_status kv_paged_attention_decode_fp8(float* out, const void* q, const void* k_pool,
                                        const void* v_pool, const int32_t* block_tables,
                                        int32_t max_blocks, const int32_t* context_lens,
                                        int32_t S, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                        float scale, kv_dtype dtype, float k_scale,
                                        float v_scale, int32_t partition_size,
                                        int32_t max_context_len, const int32_t* work_items,
                                        int32_t n_items, void* workspace, size_t ws_bytes,
                                        kv_load_policy load_policy, hipStream_t stream);

/* kv_paged_attention_decode_append over fp8 pools: the new token's K and V
 * (of `dtype`) are quantised as kv_reshape_and_cache_fp8 does and written at
 * position t-1, then attention runs as kv_paged_attention_decode_fp8. On
 * valid inputs, outputs, pools and slots are bit-identical to kv_slot_mapping
 * + kv_reshape_and_cache_fp8 + kv_paged_attention_decode_fp8. */
kv_status kv_paged_attention_decode_append_fp8(
    float* out, const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
    const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t S,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, float scale, kv_dtype dtype, float k_scale, float v_scale,
    int32_t partition_size, int32_t max_context_len, const int32_t* work_items, int32_t n_items,
    void* workspace, size_t ws_bytes, int64_t* slots, kv_load_policy load_policy,
    hipStream_t stream);

/* kv_paged_attention_decode_append_shared over fp8 pools ([1] "Memory
 * sharing" with the cache of "How does this relate to quantization?"): the
 * shared positions are read once for the batch and each sequence's tail by
 * the fp8 decode kernels, the codes widened exactly to the query's type, the
 * K scale folded into the scores and the V scale into every output before the
 * prefix ranges and the tail are combined; the new token is written as
 * kv_paged_attention_decode_append_fp8 writes it. The result is the
 * attention over positions 0..t-1 of the dequantised cache (that of
 * kv_paged_attention_decode_append_fp8 up to rounding order). Arguments,
 * checks and scratch as for kv_paged_attention_decode_append_shared, with
 * k_scale and v_scale as for kv_paged_attention_decode_append_fp8 (finite
 * and > 0, else KV_ERR_INVALID); dtype is the query's type (f16 or bf16). */
kv_status kv_paged_attention_decode_append_shared_fp8(
    float* out, const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
    const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t S,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, float scale, kv_dtype dtype, float k_scale, float v_scale,
    int32_t partition_size, int32_t shared_tokens, int32_t max_tail_len,
    const int32_t* work_items, int32_t n_items, void* workspace, size_t ws_bytes, float* aux,
    size_t aux_bytes, int64_t* slots, kv_load_policy load_policy, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Chunked prefill: several query tokens per sequence ([2] "The Successors -
 * SGLang's RadixAttention and Prefix Sharing": a prompt fed in chunks of a
 * fixed token count; [2] "Walking Through the Lifecycle", Prefill: the
 * chunk's K/V are written into the sequence's blocks).
 * ------------------------------------------------------------------------- */

/* Query rows per work item of kv_paged_attention_prefill for this head
 * configuration (0 if unsupported): 8 * (16 / G) for G = num_q_heads /
 * num_kv_heads <= 16. */
int32_t kv_paged_attention_prefill_rows_per_item(int32_t num_q_heads, int32_t num_kv_heads);

/* Work plan for kv_paged_attention_prefill from host copies of query_start
 * ([S + 1]) and context_lens ([S]): items_out receives n_items pairs
 * (sequence, row block), one per block of rows_per_item rows of each
 * sequence's chunk, the blocks whose last row sees the most keys first.
 * If cap < n_items, returns KV_ERR_INVALID with *n_items set. */
kv_status kv_paged_attention_prefill_plan(const int32_t* query_start_host,
                                          const int32_t* context_lens_host, int32_t S,
                                          int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t* items_out, int32_t cap, int32_t* n_items);

/* Attention of each sequence's chunk of query tokens over its paged cache,
 * causal within the chunk. The chunk's K and V must already be in the cache
 * (kv_slot_mapping + kv_reshape_and_cache, or kv_append_tokens).
 *
 * q:            device [total_q][num_q_heads][head_dim] of `dtype` (f16 or
 *               bf16); the rows of sequence s are query_start[s] ..
 *               query_start[s+1]-1 (C_s rows, possibly 0).
 * query_start:  device int32 [S + 1], non-decreasing, query_start[S] <= total_q.
 * context_lens: device int32 [S]: L_s cached positions of s, the chunk's
 *               included (L_s >= C_s).
 * out:          device float [total_q][num_q_heads][head_dim]: row i of
 *               sequence s (position p = L_s - C_s + i) gets
 *               sum_{j<=p} softmax_j(scale * <q, K_s[j]>) V_s[j], K_s[j] and
 *               V_s[j] read from slot(j) of KV head hq / (num_q_heads /
 *               num_kv_heads). Rows of no sequence are not written.
 * block_tables: device int32 [S][max_blocks]; k_pool / v_pool as for decode.
 * work_items:   optional device int32 [n_items][2] from
 *               kv_paged_attention_prefill_plan (grid = n_items *
 *               num_kv_heads workgroups). NULL: the grid covers S *
 *               num_kv_heads * ceil(max_query_len / rows_per_item)
 *               workgroups, max_query_len >= every C_s (host value).
 *
 * head_dim 128, group sizes 1..16, block sizes 8, 16, 32. Device-side
 * checks: a sequence with L_s < C_s or L_s > max_blocks * block_size gets
 * NaN rows; a live table entry outside [0, num_blocks) gives NaN rows and no
 * out-of-range read; a sequence whose query_start range is decreasing or
 * leaves [0, total_q] is skipped. One workgroup of 4 wave64s per item; the
 * library allocates nothing. */
kv_status kv_paged_attention_prefill(float* out, const void* q, const void* k_pool,
                                     const void* v_pool, const int32_t* block_tables,
                                     int32_t max_blocks, const int32_t* context_lens,
                                     const int32_t* query_start, int32_t S, int32_t total_q,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t block_size, int32_t num_blocks, float scale,
                                     kv_dtype dtype, int32_t max_query_len,
                                     const int32_t* work_items, int32_t n_items,
                                     hipStream_t stream);

/* kv_paged_attention_prefill over fp8 (KV_FP8_E4M3) pools with per-pool
 * scales, the cache holding value(code) * k_scale / v_scale: each code is
 * widened exactly to the query's type (`dtype`, f16 or bf16) as it is staged
 * in LDS, k_scale is folded into the score scale and v_scale into the
 * output. Write the chunk first with kv_reshape_and_cache_fp8. Arguments,
 * checks and launches otherwise as for kv_paged_attention_prefill; scales
 * must be finite and > 0 (else KV_ERR_INVALID). */
kv_status kv_paged_attention_prefill_fp8(float* out, const void* q, const void* k_pool,
                                         const void* v_pool, const int32_t* block_tables,
                                         int32_t max_blocks, const int32_t* context_lens,
                                         const int32_t* query_start, int32_t S, int32_t total_q,
                                         int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                         float scale, kv_dtype dtype, float k_scale,
                                         float v_scale, int32_t max_query_len,
                                         const int32_t* work_items, int32_t n_items,
                                         hipStream_t stream);

/* Key split for chunks that are short against their cached prefix
 * ([2] "The Custom CUDA Kernel": the partition-and-reduce of long contexts,
 * here over a block of query rows). A block's visible keys, in tiles of 32,
 * are cut into `splits` runs of equal length; each run is one workgroup per
 * KV head, which writes its rows' unnormalised sums and (max, weight sum) to
 * a workspace, and a second launch combines the runs with the online-softmax
 * rescale. Results match the unsplit call up to rounding order. */
#define KV_PREFILL_MAX_SPLITS 64

/* Number of key runs for a prefill launch from host copies of query_start
 * ([S + 1]) and context_lens ([S]): 1 when the plan's work units (items x
 * num_kv_heads) already number min_units, else the smallest count that
 * reaches min_units, capped so that the longest item keeps at least 16
 * tiles (512 keys) per run and at KV_PREFILL_MAX_SPLITS. 1 for invalid
 * arguments. */
int32_t kv_paged_attention_prefill_choose_splits(const int32_t* query_start_host,
                                                 const int32_t* context_lens_host, int32_t S,
                                                 int32_t num_q_heads, int32_t num_kv_heads,
                                                 int32_t min_units);

/* Workspace bytes kv_paged_attention_prefill_split needs: splits * total_q
 * * num_q_heads * (head_dim + 2) floats, 0 when splits <= 1 or a size is not
 * positive. The workspace needs no initialisation; calls that run
 * concurrently need separate workspaces. */
size_t kv_paged_attention_prefill_workspace_bytes(int32_t total_q, int32_t num_q_heads,
                                                 int32_t head_dim, int32_t splits);

/* kv_paged_attention_prefill with each block's keys cut into `splits` runs
 * (1..KV_PREFILL_MAX_SPLITS; 1 is the unsplit call and needs no workspace):
 * grid = items * num_kv_heads * splits workgroups, then one merge workgroup
 * per item and KV head, both on `stream`. workspace: device, 16-byte
 * aligned, at least kv_paged_attention_prefill_workspace_bytes(total_q,
 * num_q_heads, head_dim, splits) bytes, else KV_ERR_INVALID. Output, checks
 * and NaN rules as for kv_paged_attention_prefill (a NaN run makes its rows
 * NaN). */
kv_status kv_paged_attention_prefill_split(float* out, const void* q, const void* k_pool,
                                           const void* v_pool, const int32_t* block_tables,
                                           int32_t max_blocks, const int32_t* context_lens,
                                           const int32_t* query_start, int32_t S, int32_t total_q,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int32_t num_blocks, float scale, kv_dtype dtype,
                                           int32_t max_query_len, const int32_t* work_items,
                                           int32_t n_items, int32_t splits, void* workspace,
                                           size_t ws_bytes, hipStream_t stream);

/* kv_paged_attention_prefill_split over fp8 pools, scales as for
 * kv_paged_attention_prefill_fp8. */
kv_status kv_paged_attention_prefill_split_fp8(
    float* out, const void* q, const void* k_pool, const void* v_pool,
    const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
    const int32_t* query_start, int32_t S, int32_t total_q, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    kv_dtype dtype, float k_scale, float v_scale, int32_t max_query_len,
    const int32_t* work_items, int32_t n_items, int32_t splits, void* workspace, size_t ws_bytes,
    hipStream_t stream);

/* Message describing the calling thread's last error ("" if none). */
const char* kv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H_ */
