"""Oracle for the host block manager: free list, refcounts, sequences.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Pages cited in this file:
  [1] "PagedAttention - how vLLM stopped wasting 80% of your GPU memory"
      (shivam2003.com/posts/pagedattention.html)
  [2] "PagedAttention: How vLLM Borrowed Virtual Memory to Unlock GPU Serving
      at Scale" (fp4-site.pages.dev/system/pagedattention-vllm-deep-dive/)
  [3] "PagedAttention and vLLM: Virtual Memory for the KV Cache" (passgenai.com)
  [4] "What is paged attention?" (netraruntime.com/learn/paged-attention)

What the pages fix:
  * a fixed pool of uniform blocks; capacity is num_blocks * block_size tokens
    ([3], "L2 - Mechanism", the block pool);
  * taking a block pops the free list and returning one pushes it, both O(1);
    a sequence of t tokens holds ceil(t / B) blocks ([4], "How it works");
  * every physical block carries a reference count; a fork points the child
    at the parent's blocks ([1], "Memory sharing"; [3], copy-on-write);
  * writing into a block whose count exceeds one first copies it into a new
    block, drops the old block's count and redirects the writer ([2],
    "Copy-on-Write ..."); appending after a full shared block copies nothing
    ([1], "A small worked example", step 3);
  * a finished sequence returns every block ([2], "Sequence Completion");
  * under memory pressure a sequence can be preempted by swapping its blocks
    to host memory and bringing them back when it is readmitted ([3], "The
    allocation lifecycle", memory pressure; [1], "Preemption"), all or
    nothing per sequence ([3], "L3").

Readings where the pages leave a choice open:
  * growth is lazy: a new block is taken just before writing position p when
    p mod B == 0, which is the only reading that keeps ceil(t / B) blocks;
  * the free list is a LIFO stack. Its initial content is given as an order
    whose first element is handed out first ([1]'s example hands out P0, P1
    first); freeing pushes a sequence's blocks in reverse logical order so a
    re-allocation returns them in logical order ([1]'s example reuses P0, P1
    for request C);
  * copy-on-write happens only when the written block's count exceeds one;
    it copies the whole block; it allocates the copy before any new block of
    the same append;
  * every operation is all-or-nothing: on failure nothing changes ([3], "L3",
    preemption is all-or-nothing per sequence);
  * swapping out returns the sequence's current table (the blocks whose
    contents go to host memory, in logical order) and then drops one
    reference per block exactly as freeing does; the sequence keeps its
    length. Swapping in takes ceil(length / B) fresh blocks (reference count
    1, popped in logical order) that the contents are copied back into; a
    block shared with another sequence before the swap comes back as a
    private copy. A swapped-out sequence cannot be appended to, forked or
    packed until it is swapped back in; it can be freed.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple


class KVError(Exception):
    """Failure with the status name the C ABI uses (INVALID, OOM, STATE)."""

    def __init__(self, code: str, msg: str = ""):
        super().__init__(f"{code}: {msg}")
        self.code = code


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int = 16,
                 free_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise KVError("INVALID", "pool sizes must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.refcount = [0] * num_blocks
        order = list(range(num_blocks)) if free_order is None else [int(x) for x in free_order]
        self._set_stack(order)
        self.tables: Dict[int, List[int]] = {}
        self.lengths: Dict[int, int] = {}
        self.swapped: set = set()
        self._next_seq = 0

    # -- pool ---------------------------------------------------------------
    def _set_stack(self, order: List[int]) -> None:
        if sorted(order) != list(range(self.num_blocks)):
            raise KVError("INVALID", "free order must be a permutation of all block IDs")
        # top of the stack is the end of the list; order[0] must pop first
        self.free = list(reversed(order))

    def set_free_order(self, order: Sequence[int]) -> None:
        if any(self.refcount):
            raise KVError("STATE", "free order can only be set while every block is free")
        self._set_stack([int(x) for x in order])

    def capacity_tokens(self) -> int:
        return self.num_blocks * self.block_size

    def num_free(self) -> int:
        return len(self.free)

    def alloc(self, n: int) -> List[int]:
        if n < 0:
            raise KVError("INVALID", "negative count")
        if n > len(self.free):
            raise KVError("OOM", f"need {n} blocks, {len(self.free)} free")
        ids = [self.free.pop() for _ in range(n)]
        for b in ids:
            self.refcount[b] = 1
        return ids

    def _check_held(self, ids: Sequence[int], decrement: bool) -> None:
        need: Dict[int, int] = {}
        for b in ids:
            if not (0 <= b < self.num_blocks):
                raise KVError("INVALID", f"block {b} outside the pool")
            need[b] = need.get(b, 0) + 1
        for b, c in need.items():
            if self.refcount[b] == 0 or (decrement and self.refcount[b] < c):
                raise KVError("STATE", f"block {b} is not held")

    def incref(self, ids: Sequence[int]) -> None:
        ids = [int(b) for b in ids]
        self._check_held(ids, decrement=False)
        for b in ids:
            self.refcount[b] += 1

    def decref(self, ids: Sequence[int]) -> None:
        """Drop one reference per listed block; push blocks that reach zero,
        in reverse list order so that list order is the next pop order."""
        ids = [int(b) for b in ids]
        self._check_held(ids, decrement=True)
        for b in reversed(ids):
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)

    # -- sequences ----------------------------------------------------------
    def _seq(self, seq: int) -> List[int]:
        if seq not in self.tables:
            raise KVError("STATE", f"unknown sequence {seq}")
        if seq in self.swapped:
            raise KVError("STATE", f"sequence {seq} is swapped out")
        return self.tables[seq]

    def create(self) -> int:
        sid = self._next_seq
        self._next_seq += 1
        self.tables[sid] = []
        self.lengths[sid] = 0
        return sid

    def fork(self, parent: int) -> int:
        table = self._seq(parent)
        self.incref(table)
        sid = self.create()
        self.tables[sid] = list(table)
        self.lengths[sid] = self.lengths[parent]
        return sid

    def append(self, seq: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Reserve slots for n new tokens of `seq`.

        Returns (slots, cow_pairs): the physical slot of each new position and
        the (src, dst) block copies the device must perform before writing.
        """
        table = self._seq(seq)
        if n < 0:
            raise KVError("INVALID", "negative token count")
        B = self.block_size
        t = self.lengths[seq]
        if n == 0:
            return [], []
        have = -(-t // B)
        need_new = -(-(t + n) // B) - have
        cow = t % B != 0 and self.refcount[table[-1]] > 1
        if need_new + (1 if cow else 0) > len(self.free):
            raise KVError("OOM", "not enough free blocks for the append")
        pairs: List[Tuple[int, int]] = []
        if cow:
            src = table[-1]
            dst = self.free.pop()
            self.refcount[dst] = 1
            self.refcount[src] -= 1
            table[-1] = dst
            pairs.append((src, dst))
        for _ in range(need_new):
            b = self.free.pop()
            self.refcount[b] = 1
            table.append(b)
        slots = []
        for p in range(t, t + n):
            slots.append(table[p // B] * B + p % B)
        self.lengths[seq] = t + n
        return slots, pairs

    def free_seq(self, seq: int) -> None:
        if seq in self.swapped:  # holds no blocks
            self.swapped.discard(seq)
        else:
            self.decref(self._seq(seq))
        del self.tables[seq]
        del self.lengths[seq]

    def swap_out(self, seq: int) -> List[int]:
        """Preempt `seq`: return its table, then release its blocks."""
        table = list(self._seq(seq))
        self.decref(table)
        self.tables[seq] = []
        self.swapped.add(seq)
        return table

    def swap_in(self, seq: int) -> List[int]:
        """Readmit `seq`: ceil(length / B) fresh blocks, all or nothing."""
        if seq not in self.tables:
            raise KVError("STATE", f"unknown sequence {seq}")
        if seq not in self.swapped:
            raise KVError("STATE", f"sequence {seq} is not swapped out")
        need = -(-self.lengths[seq] // self.block_size)
        ids = self.alloc(need)
        self.tables[seq] = list(ids)
        self.swapped.discard(seq)
        return list(ids)

    def is_swapped(self, seq: int) -> bool:
        if seq not in self.tables:
            raise KVError("STATE", f"unknown sequence {seq}")
        return seq in self.swapped

    def table(self, seq: int) -> List[int]:
        return list(self._seq(seq))

    def length(self, seq: int) -> int:
        if seq not in self.lengths:
            raise KVError("STATE", f"unknown sequence {seq}")
        return self.lengths[seq]

    # -- helpers for tests --------------------------------------------------
    def packed_tables(self, seqs: Sequence[int], max_blocks: Optional[int] = None,
                      pad: int = -1):
        """[len(seqs), max_blocks] table array padded with `pad`, and lengths."""
        import numpy as np
        tabs = [self.table(s) for s in seqs]
        width = max_blocks if max_blocks is not None else max([len(t) for t in tabs] + [1])
        out = np.full((len(seqs), width), pad, dtype=np.int32)
        for i, t in enumerate(tabs):
            out[i, :len(t)] = t
        lens = np.array([self.lengths[s] for s in seqs], dtype=np.int32)
        return out, lens


def run_ops(bm: BlockManager, ops, handles: Optional[Dict[int, int]] = None):
    """Apply a workload operation script; returns (handles, slots_by_op,
    cow_pairs) where handles maps script sequence numbers to manager IDs."""
    handles = {} if handles is None else handles
    all_slots = []
    all_pairs = []
    for op in ops:
        if op[0] == "create":
            handles[op[1]] = bm.create()
            all_slots.append(None)
        elif op[0] == "fork":
            handles[op[2]] = bm.fork(handles[op[1]])
            all_slots.append(None)
        elif op[0] == "append":
            slots, pairs = bm.append(handles[op[1]], op[2])
            all_slots.append(slots)
            all_pairs.extend(pairs)
        else:
            raise ValueError(op)
    return handles, all_slots, all_pairs
