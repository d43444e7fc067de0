"""One layer's paged KV cache on the GPU and the decode step over it.

DecodeSession ties the host block manager (libpagedkv's kv_pool_* / kv_seq_*)
to device buffers owned by torch, and runs the decode step as the pages'
lifecycle describes it ("PagedAttention and vLLM: Virtual Memory for the KV
Cache", passgenai.com, "The allocation lifecycle"): reserve a slot for each
sequence's new token, write the token's K/V into it, then attend over the
whole cache. The host part (`prepare_step`) and the device part (`step`) are
separate so a benchmark can time the device part alone.

Operation scripts are lists of tuples: ("create", s), ("fork", parent, child),
("append", s, n), ("free", s) where s are caller-chosen sequence numbers.

Pools of dtype uint8 are an fp8 (E4M3) cache: every write quantises with the
session's k_scale / v_scale and attention goes through the _fp8 entry points.

When every sequence of a decode step reaches its first positions through the
same blocks (a shared prefix: "PagedAttention - how vLLM stopped wasting 80% of
your GPU memory", "Memory sharing"), the step
goes through kv_paged_attention_decode_append_shared, which reads those blocks
once for the batch instead of once per sequence (shared_prefix=False turns
this off).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import binding as kv

# Work units below which a longer partition is not chosen: about 3/4 of the
# 2048 waves an MI355X runs at once (256 CUs x 8 waves), measured best.
AUTO_PARTITION_MIN_UNITS = 1500
MI355X_CUS = 256
# Prefill workgroups (4 waves each) per compute unit below which a chunk's
# keys are split into runs: two fill a CU at the kernel's register use.
PREFILL_UNITS_PER_CU = 2

class DecodeSession:
    def __init__(self, *, k_pool, v_pool, num_q_heads: int, free_order: Optional[Sequence[int]] = None,
                 partition_size: int = 0, use_plan: bool = True, fused: bool = True,
                 k_scale: float = 1.0, v_scale: float = 1.0, shared_prefix: bool = True,
                 num_cus: Optional[int] = None, prefill_splits: Optional[int] = None):
        import torch
        self.torch = torch
        NB, Hkv, B, D = k_pool.shape
        self.k_pool, self.v_pool = k_pool, v_pool
        self.NB, self.Hkv, self.B, self.D, self.Hq = NB, Hkv, B, D, num_q_heads
        self.dtype = kv.dtype_code(k_pool)
        self.fp8 = self.dtype == kv.KV_FP8_E4M3
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)
        # 0: choose per step from the batch's lengths (the library's own
        # default, 512 tokens, is what the entry points use for 0)
        self.partition_size = partition_size
        self.min_units = AUTO_PARTITION_MIN_UNITS
        self.use_plan = use_plan
        self.fused = fused
        # decode steps over a common prefix read it once (fused 16-bit steps only)
        self.shared_prefix = shared_prefix
        self.shared_tokens = 0
        self.pool = kv.kv_pool_create(NB, B, 1, Hkv, D, self.dtype)
        if free_order is not None:
            kv.kv_pool_set_free_order(self.pool, free_order)
        self.handles: Dict[int, int] = {}
        self.block_bytes = Hkv * B * D * k_pool.element_size()
        self.device = k_pool.device
        # compute units the decode plan lays its work out for (host-only
        # sessions on CPU tensors plan for an MI355X's 256)
        if num_cus is None:
            num_cus = (torch.cuda.get_device_properties(self.device).multi_processor_count
                       if self.device.type == "cuda" else MI355X_CUS)
        self.num_cus = int(num_cus)
        # key runs per prefill block: None chooses per step
        # (kv_paged_attention_prefill_choose_splits), else a fixed count
        self.prefill_splits = prefill_splits
        self.step_splits = 1
        self.d_prefill_ws = None

    def close(self) -> None:
        if self.pool:
            kv.kv_pool_destroy(self.pool)
            self.pool = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- host operations (plus the device writes they imply) ----------------
    def run_ops(self, ops, values: Optional[Dict[int, Tuple]] = None) -> List[Tuple[int, int]]:
        """Apply an operation script. Copy-on-write pairs reported by an
        append are copied on the device at once. An append tagged "values"
        (4th element) then writes values[s] = (k, v), device tensors
        [n, Hkv, D], into the new slots. Returns the copy-on-write pairs."""
        torch = self.torch
        cows: List[Tuple[int, int]] = []
        for op in ops:
            if op[0] == "create":
                self.handles[op[1]] = kv.kv_seq_create(self.pool)
            elif op[0] == "fork":
                self.handles[op[2]] = kv.kv_seq_fork(self.pool, self.handles[op[1]])
            elif op[0] == "free":
                kv.kv_seq_free(self.pool, self.handles.pop(op[1]))
            elif op[0] == "append":
                s, n = op[1], op[2]
                slots, pair = kv.kv_seq_append(self.pool, self.handles[s], n)
                if pair is not None:
                    cows.append(pair)
                    p = torch.tensor([pair], dtype=torch.int32, device=self.device)
                    kv.kv_copy_blocks([self.k_pool], [self.v_pool], p, self.NB, self.block_bytes)
                if len(op) > 3 and op[3] == "values":
                    k, v = values[s]
                    d_slots = torch.from_numpy(slots).to(self.device)
                    self._write(k, v, self.k_pool, self.v_pool, d_slots)
            else:
                raise ValueError(op)
        return cows

    # -- preemption by swapping ([3], "The allocation lifecycle", memory
    # pressure; [1], "Preemption") ------------------------------------------
    def swap_out(self, s: int):
        """Move sequence s's blocks to a new pinned host buffer and release
        them to the pool. The copy is queued on the current stream; device
        writes into the released blocks that later calls queue on the same
        stream run after it. Returns the buffer ([blocks][K, V][block bytes])
        that swap_in needs."""
        torch = self.torch
        ids = kv.kv_seq_swap_out(self.pool, self.handles[s])
        host = torch.empty(max(len(ids), 1) * 2 * self.block_bytes, dtype=torch.uint8,
                           pin_memory=True)
        if len(ids):
            d_ids = torch.from_numpy(ids).to(self.device)
            kv.kv_swap_out_blocks([self.k_pool], [self.v_pool], d_ids, self.NB, self.block_bytes,
                                  host)
            self._keep_until_done(host, d_ids)
        return host

    def swap_in(self, s: int, host) -> np.ndarray:
        """Readmit sequence s: take fresh blocks (all or nothing) and copy the
        swap_out buffer into them on the current stream. Returns the blocks."""
        torch = self.torch
        ids = kv.kv_seq_swap_in(self.pool, self.handles[s])
        if len(ids):
            d_ids = torch.from_numpy(ids).to(self.device)
            kv.kv_swap_in_blocks([self.k_pool], [self.v_pool], d_ids, self.NB, self.block_bytes,
                                 host)
            self._keep_until_done(host, d_ids)
        return ids

    def _keep_until_done(self, *tensors) -> None:
        # the kernels use raw pointers, which torch's allocators do not track:
        # hold the buffers until an event behind the copy has completed
        pending = getattr(self, "_pending", [])
        pending = [(e, t) for e, t in pending if not e.query()]
        ev = self.torch.cuda.Event()
        ev.record()
        pending.append((ev, tensors))
        self._pending = pending

    def _write(self, k, v, kp, vp_, d_slots) -> None:
        if self.fp8:
            kv.kv_reshape_and_cache_fp8(k, v, kp, vp_, d_slots, self.k_scale, self.v_scale)
        else:
            kv.kv_reshape_and_cache(k, v, kp, vp_, d_slots)

    def tables(self, seqs: Sequence[int], max_blocks: Optional[int] = None):
        ids = [self.handles[s] for s in seqs]
        if max_blocks is None:
            max_blocks = max(1, max(-(-kv.kv_seq_len(self.pool, h) // self.B) for h in ids))
        return kv.kv_seq_pack_tables(self.pool, ids, max_blocks)

    # -- a chunked-prefill step ----------------------------------------------
    def prepare_prefill(self, seqs: Sequence[int], counts: Sequence[int]):
        """Host half of a chunked-prefill step: reserve counts[i] new positions
        for sequence seqs[i] and upload the slots, tables, lengths, query row
        ranges and the work plan. Returns the host-side slots and any
        copy-on-write pairs."""
        torch = self.torch
        dev = self.device
        slots, pairs = [], []
        for s, n in zip(seqs, counts):
            sl, pair = kv.kv_seq_append(self.pool, self.handles[s], int(n))
            slots.append(sl)
            if pair is not None:
                pairs.append(pair)
        host_slots = np.concatenate(slots).astype(np.int64) if slots else np.zeros(0, np.int64)
        tables, lens = self.tables(seqs)
        q_start = np.concatenate([[0], np.cumsum(np.asarray(counts, np.int64))]).astype(np.int32)
        self.seqs = list(seqs)
        self.d_tables = torch.from_numpy(tables).to(dev)
        self.d_lens = torch.from_numpy(lens).to(dev)
        self.d_qstart = torch.from_numpy(q_start).to(dev)
        self.d_slots = torch.from_numpy(host_slots).to(dev)
        self.d_pairs = torch.tensor(pairs, dtype=torch.int32, device=dev).reshape(-1, 2)
        self.max_query_len = int(max(counts)) if len(counts) else 0
        self.host_tables, self.host_lens, self.host_qstart = tables, lens, q_start
        self.d_items = None
        if self.use_plan:
            items = kv.kv_paged_attention_prefill_plan(q_start, lens, self.Hq, self.Hkv)
            self.d_items = torch.from_numpy(items).to(dev) if len(items) else None
        self.step_splits = self.prefill_splits or kv.kv_paged_attention_prefill_choose_splits(
            q_start, lens, self.Hq, self.Hkv, PREFILL_UNITS_PER_CU * self.num_cus)
        need = kv.kv_paged_attention_prefill_workspace_bytes(int(q_start[-1]), self.Hq, self.D,
                                                             self.step_splits)
        if need and (self.d_prefill_ws is None or self.d_prefill_ws.numel() < need):
            self.d_prefill_ws = torch.empty(need, dtype=torch.uint8, device=dev)
        return host_slots, pairs

    def prefill_step(self, q, k_new, v_new, out, scale: float, k_pool=None, v_pool=None,
                     events=None) -> None:
        """Device half of a chunked-prefill step on the current stream:
        copy-on-write copies (if any), the chunk's K/V written into its slots,
        then the causal attention of every chunk row. `events` = (start, end)
        torch events recorded around the attention launch."""
        kp = self.k_pool if k_pool is None else k_pool
        vp_ = self.v_pool if v_pool is None else v_pool
        if self.d_pairs.shape[0]:
            kv.kv_copy_blocks([kp], [vp_], self.d_pairs, self.NB, self.block_bytes)
        self._write(k_new, v_new, kp, vp_, self.d_slots)
        if events is not None:
            events[0].record()
        if self.step_splits > 1 and self.fp8:
            kv.kv_paged_attention_prefill_split_fp8(out, q, kp, vp_, self.d_tables, self.d_lens,
                                                    self.d_qstart, scale, self.k_scale,
                                                    self.v_scale, self.max_query_len,
                                                    self.step_splits, self.d_prefill_ws,
                                                    self.d_items)
        elif self.step_splits > 1:
            kv.kv_paged_attention_prefill_split(out, q, kp, vp_, self.d_tables, self.d_lens,
                                                self.d_qstart, scale, self.max_query_len,
                                                self.step_splits, self.d_prefill_ws,
                                                self.d_items)
        elif self.fp8:
            kv.kv_paged_attention_prefill_fp8(out, q, kp, vp_, self.d_tables, self.d_lens,
                                              self.d_qstart, scale, self.k_scale, self.v_scale,
                                              self.max_query_len, self.d_items)
        else:
            kv.kv_paged_attention_prefill(out, q, kp, vp_, self.d_tables, self.d_lens,
                                          self.d_qstart, scale, self.max_query_len, self.d_items)
        if events is not None:
            events[1].record()

    # -- the decode step ----------------------------------------------------
    def prepare_step(self, seqs: Sequence[int]):
        """Host half of a decode step: reserve one new slot per sequence and
        upload tables, lengths and the (sequence, position) list. Returns the
        host-side slots the allocator chose and any copy-on-write pairs."""
        torch = self.torch
        host_slots = np.zeros(len(seqs), dtype=np.int64)
        pairs = []
        for i, s in enumerate(seqs):
            sl, pair = kv.kv_seq_append(self.pool, self.handles[s], 1)
            host_slots[i] = sl[0]
            if pair is not None:
                pairs.append(pair)
        tables, lens = self.tables(seqs)
        dev = self.device
        S = len(seqs)
        self.shared_tokens = self._common_prefix_tokens(tables, lens)
        # the decode kernels see the tails of a shared-prefix step, else everything
        dlens = lens - self.shared_tokens
        # (short tails measured fastest with the same 512-token floor as
        # whole sequences: smaller partitions add a merge launch)
        self.step_partition = self.partition_size or kv.kv_paged_attention_choose_partition(
            dlens, self.Hkv, self.B, self.min_units)
        self.seqs = list(seqs)
        self.d_tables = torch.from_numpy(tables).to(dev)
        self.d_lens = torch.from_numpy(lens).to(dev)
        self.d_seq_idx = torch.arange(len(seqs), dtype=torch.int32, device=dev)
        self.d_pos = (self.d_lens - 1).contiguous()
        self.d_slots = torch.empty(len(seqs), dtype=torch.int64, device=dev)
        self.d_pairs = torch.tensor(pairs, dtype=torch.int32, device=dev).reshape(-1, 2)
        self.max_context_len = int(lens.max()) if len(lens) else 0
        self.max_decode_len = int(dlens.max()) if len(dlens) else 0
        ws = kv.kv_paged_attention_workspace_bytes(S, self.Hq, self.Hkv, self.D,
                                                   self.max_decode_len, self.step_partition)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev) if ws else None
        self.aux = None
        if self.shared_tokens:
            aux = kv.kv_paged_attention_shared_aux_bytes(S, self.Hq, self.Hkv, self.D,
                                                         self.shared_tokens)
            self.aux = torch.empty(aux // 4, dtype=torch.float32, device=dev)
        self.host_tables, self.host_lens = tables, lens
        self.d_items = None
        if self.use_plan:
            items = kv.kv_paged_attention_plan(dlens, self.step_partition, self.Hkv, self.num_cus)
            self.d_items = torch.from_numpy(items).to(dev)
        # blocks the decode kernels read for several sequences in the step
        # stay in the caches; otherwise every block streams past them (the
        # shared prefix of a shared-prefix step is read once, elsewhere)
        self.load_policy = kv.kv_paged_attention_choose_load_policy(self.pool, self.shared_tokens)
        return host_slots, pairs

    def _common_prefix_tokens(self, tables, lens) -> int:
        """Positions the step's shared-prefix entry point treats as common: the
        library's choice for the batch (kv_paged_attention_choose_shared_prefix:
        the common leading blocks where that step applies and is expected to
        pay), or 0 when the session runs plain steps (shared_prefix=False) or
        unfused steps, which the shared-prefix entry point does not offer."""
        if not self.shared_prefix or not self.fused:
            return 0
        return kv.kv_paged_attention_choose_shared_prefix(tables, lens, self.B, self.Hq, self.Hkv,
                                                          self.D, self.dtype)

    def write_step_tokens(self, k_new, v_new, k_pool=None, v_pool=None) -> None:
        """The unfused cache write of the step on its own: slot mapping of
        every new token and the write of its K/V rows (one launch for a
        16-bit cache, two for fp8), on the current stream."""
        kp = self.k_pool if k_pool is None else k_pool
        vp_ = self.v_pool if v_pool is None else v_pool
        if self.fp8:
            kv.kv_slot_mapping(self.d_tables, self.d_seq_idx, self.d_pos, self.d_slots, self.B)
            self._write(k_new, v_new, kp, vp_, self.d_slots)
        else:
            kv.kv_append_tokens(self.d_tables, self.d_seq_idx, self.d_pos, k_new, v_new, kp, vp_,
                                self.d_slots)

    def step(self, q, k_new, v_new, out, scale: float, k_pool=None, v_pool=None,
             decode_events=None, fused: Optional[bool] = None) -> None:
        """Device half of a decode step, all on the current stream:
        copy-on-write copies (if any), then either the fused decode (cache
        write + attention, one launch plus the split-K merge; for a step over
        a common prefix, the shared-prefix decode: tails, prefix once, and
        their combination) or, with fused=False, slot mapping + cache write
        (one launch) followed by the decode. `decode_events` = (start, end) torch events recorded around
        the call that runs attention."""
        kp = self.k_pool if k_pool is None else k_pool
        vp_ = self.v_pool if v_pool is None else v_pool
        fused = self.fused if fused is None else fused
        if self.shared_tokens and not fused:
            raise ValueError("this step was prepared for the shared-prefix decode, which fuses "
                             "the cache write; create the session with shared_prefix=False")
        if self.d_pairs.shape[0]:
            kv.kv_copy_blocks([kp], [vp_], self.d_pairs, self.NB, self.block_bytes)
        if not fused:
            self.write_step_tokens(k_new, v_new, kp, vp_)
        if decode_events is not None:
            decode_events[0].record()
        if self.fp8 and self.shared_tokens:
            kv.kv_paged_attention_decode_append_shared_fp8(
                out, q, k_new, v_new, kp, vp_, self.d_tables, self.d_lens, scale, self.k_scale,
                self.v_scale, self.shared_tokens, self.max_decode_len, self.d_slots, self.aux,
                self.workspace, self.step_partition, self.d_items, load_policy=self.load_policy)
        elif self.fp8:
            if fused:
                kv.kv_paged_attention_decode_append_fp8(
                    out, q, k_new, v_new, kp, vp_, self.d_tables, self.d_lens, scale, self.k_scale,
                    self.v_scale, self.max_context_len, self.d_slots, self.workspace,
                    self.step_partition, self.d_items, load_policy=self.load_policy)
            else:
                kv.kv_paged_attention_decode_fp8(
                    out, q, kp, vp_, self.d_tables, self.d_lens, scale, self.k_scale, self.v_scale,
                    self.max_context_len, self.workspace, self.step_partition, self.d_items,
                    load_policy=self.load_policy)
        elif self.shared_tokens:
            kv.kv_paged_attention_decode_append_shared(
                out, q, k_new, v_new, kp, vp_, self.d_tables, self.d_lens, scale,
                self.shared_tokens, self.max_decode_len, self.d_slots, self.aux, self.workspace,
                self.step_partition, self.d_items, load_policy=self.load_policy)
        elif fused:
            kv.kv_paged_attention_decode_append(out, q, k_new, v_new, kp, vp_, self.d_tables,
                                                self.d_lens, scale, self.max_context_len,
                                                self.d_slots, self.workspace, self.step_partition,
                                                self.d_items, load_policy=self.load_policy)
        else:
            kv.kv_paged_attention_decode(out, q, kp, vp_, self.d_tables, self.d_lens, scale,
                                         self.max_context_len, self.workspace, self.step_partition,
                                         self.d_items, load_policy=self.load_policy)
        if decode_events is not None:
            decode_events[1].record()
