"""Oracle for the device-side steps of paged decode attention (float64 numpy).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Pages cited in this file:
  [1] "PagedAttention - how vLLM stopped wasting 80% of your GPU memory"
      (shivam2003.com/posts/pagedattention.html)
  [2] "PagedAttention: How vLLM Borrowed Virtual Memory to Unlock GPU Serving
      at Scale" (fp4-site.pages.dev/system/pagedattention-vllm-deep-dive/)
  [3] "PagedAttention and vLLM: Virtual Memory for the KV Cache" (passgenai.com)
  [4] "What is paged attention?" (netraruntime.com/learn/paged-attention)

Layout (from [2], "The Custom CUDA Kernel"): each layer has a K pool and a V
pool of shape [num_blocks, num_kv_heads, block_size, head_dim]; the leading
index is the physical block ID. The query is [num_seqs, num_q_heads, head_dim];
block tables are [num_seqs, max_blocks] int32; context lengths are [num_seqs].

Readings where the pages leave a step open:
  * positions p >= context_len inside the last block are excluded from the
    softmax ([1]'s kernel sketch softmaxes whole blocks; [2] passes the actual
    lengths and [3] calls the last block partially filled);
  * scores are multiplied by an explicit `scale` (absent from [1]'s sketch);
  * grouped-query attention maps query head hq to KV head hq // (Hq // Hkv);
  * a sequence of length 0 attends to nothing and its output is 0.

Storage dtypes arrive as numpy arrays: float32, float16, uint16 holding bf16
bit patterns, or uint8 holding fp8 E4M3 codes (see oracle/fp8.py). They are
widened exactly to float64 before any arithmetic.
"""
from __future__ import annotations

from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact conversion of stored values to float64.

    bf16 is the upper 16 bits of an IEEE binary32 encoding, so the widening
    places the stored bits in the high half of a 32-bit word.
    """
    x = np.asarray(x)
    if dtype == "bf16":
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype in ("f32", "f16"):
        return x.astype(np.float64)
    if dtype == "e4m3":
        from .fp8 import e4m3_decode
        return e4m3_decode(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def slot_of(table_row: Sequence[int], p: int, block_size: int = 16) -> int:
    """Physical slot of logical position p ([4], "How it works"): the block
    table entry of logical block floor(p / B), times B, plus p mod B."""
    return int(table_row[p // block_size]) * block_size + p % block_size


def slot_mapping(tables: np.ndarray, seq_idx: np.ndarray, pos: np.ndarray,
                 block_size: int = 16) -> np.ndarray:
    """Slot of each (sequence, position) pair, as int64.

    Entries that cannot be mapped (negative position, logical block beyond the
    table width, or a negative table entry) give -1, which the cache scatter
    skips. One Python loop per entry keeps every case visible.
    """
    tables = np.asarray(tables)
    max_blocks = tables.shape[1]
    out = np.empty(len(pos), dtype=np.int64)
    for i, (s, p) in enumerate(zip(seq_idx, pos)):
        s, p = int(s), int(p)
        if p < 0 or p // block_size >= max_blocks:
            out[i] = -1
            continue
        entry = int(tables[s, p // block_size])
        out[i] = -1 if entry < 0 else slot_of(tables[s], p, block_size)
    return out


def gather_sequence(pool: np.ndarray, table_row: Sequence[int], ctx: int,
                    block_size: int = 16) -> np.ndarray:
    """Rebuild a sequence's contiguous cache [ctx, Hkv, D] position by position
    through the slot formula ([4], "How it works"), in storage dtype."""
    num_blocks = pool.shape[0]
    nb = -(-ctx // block_size)
    for i in range(nb):
        if not (0 <= int(table_row[i]) < num_blocks):
            raise ValueError(f"block table entry {i} = {table_row[i]} outside the pool")
    rows = []
    for p in range(ctx):
        s = slot_of(table_row, p, block_size)
        rows.append(pool[s // block_size, :, s % block_size, :])
    if not rows:
        return pool[:0, :, 0, :]
    return np.stack(rows, axis=0)


def _kv_head(hq: int, Hq: int, Hkv: int) -> int:
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    return hq // (Hq // Hkv)


def decode_attention(q, k_pool, v_pool, block_tables, context_lens, scale: float,
                     dtype: str, block_size: int = 16,
                     pairs: Optional[Iterable[Tuple[int, int]]] = None,
                     kv_dtype: Optional[str] = None, k_scale: float = 1.0,
                     v_scale: float = 1.0) -> np.ndarray:
    """Decode attention over a paged cache, as the plain definition.

    [1] ("The PagedAttention kernel") states that walking the block table
    produces exactly the attention of a contiguous cache, with no
    approximation. So for each sequence s the cache is first rebuilt in
    logical order, then out[s, hq] = sum_j w_j V[j] / sum_j w_j with
    w_j = exp(z_j - max z), z_j = scale * <q[s, hq], K[j]>, j < ctx.

    Returns float64 [S, Hq, D]. With `pairs`, only those (s, hq) entries are
    computed and the rest stay NaN. `kv_dtype` is the pools' storage type when
    it differs from the query's (an fp8 cache, "e4m3"); the cache then holds
    code value times `k_scale` (K) or `v_scale` (V).
    """
    q = widen(q, dtype)
    S, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    out = np.full((S, Hq, D), np.nan)
    if pairs is None:
        pairs = [(s, h) for s in range(S) for h in range(Hq)]
    by_seq = {}
    for s, h in pairs:
        by_seq.setdefault(int(s), []).append(int(h))
    sc = float(np.float64(scale))
    for s, heads in by_seq.items():
        ctx = int(context_lens[s])
        if ctx == 0:
            out[s, heads] = 0.0
            continue
        kd = kv_dtype or dtype
        Kc = widen(gather_sequence(k_pool, block_tables[s], ctx, block_size), kd)
        Vc = widen(gather_sequence(v_pool, block_tables[s], ctx, block_size), kd)
        if kv_dtype is not None:
            Kc = Kc * float(np.float32(k_scale))
            Vc = Vc * float(np.float32(v_scale))
        for hq in heads:
            h = _kv_head(hq, Hq, Hkv)
            z = sc * (Kc[:, h, :] @ q[s, hq])
            w = np.exp(z - z.max())
            out[s, hq] = (w @ Vc[:, h, :]) / w.sum()
    return out


def decode_attention_blockwise(q, k_pool, v_pool, block_tables, context_lens,
                               scale: float, dtype: str, block_size: int = 16) -> np.ndarray:
    """A second loop order, block by block, as [1]'s kernel sketch walks it.

    For every logical block the physical block is fetched whole and scored
    against the query; the concatenated scores are softmaxed over all
    positions; the output is the sum over blocks of the block's weights times
    its V rows. Masking of positions >= ctx and the scale are added. This path
    never evaluates the slot formula: it indexes whole physical blocks.
    """
    q = widen(q, dtype)
    S, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    out = np.zeros((S, Hq, D))
    sc = float(np.float64(scale))
    for s in range(S):
        ctx = int(context_lens[s])
        if ctx == 0:
            continue
        nb = -(-ctx // block_size)
        for hq in range(Hq):
            h = _kv_head(hq, Hq, Hkv)
            scores = []
            for logical in range(nb):
                phys = int(block_tables[s][logical])
                kb = widen(k_pool[phys, h], dtype)            # [B, D]
                scores.append(sc * (kb @ q[s, hq]))
            z = np.concatenate(scores)
            valid = np.arange(nb * block_size) < ctx
            zmax = z[valid].max()
            w = np.where(valid, np.exp(np.where(valid, z, zmax) - zmax), 0.0)
            w = w / w.sum()
            acc = np.zeros(D)
            for logical in range(nb):
                phys = int(block_tables[s][logical])
                vb = widen(v_pool[phys, h], dtype)
                wb = w[logical * block_size:(logical + 1) * block_size]
                keep = valid[logical * block_size:(logical + 1) * block_size]
                acc += wb[keep] @ vb[keep]
            out[s, hq] = acc
    return out


def partial_attention(Kc: np.ndarray, Vc: np.ndarray, qv: np.ndarray, scale: float):
    """Unnormalised partial result of one context partition: (m, l, o) with
    m = max z, l = sum exp(z - m), o = sum exp(z - m) V (float64)."""
    z = float(scale) * (Kc @ qv)
    m = z.max()
    w = np.exp(z - m)
    return m, w.sum(), w @ Vc


def merge_partials(parts: List[Tuple[float, float, np.ndarray]]) -> np.ndarray:
    """Numerically stable merge of per-partition results ([2], "The Custom
    CUDA Kernel": partial outputs and softmax denominators are computed per
    piece and then combined). The page does not print the formula; the
    log-sum-exp merge is used: M = max m_k, L = sum l_k e^(m_k - M),
    out = sum e^(m_k - M) o_k / L."""
    M = max(m for m, _, _ in parts)
    L = sum(l * np.exp(m - M) for m, l, _ in parts)
    O = sum(np.exp(m - M) * o for m, _, o in parts)
    return O / L


def decode_attention_split(q, k_pool, v_pool, block_tables, context_lens, scale: float,
                           dtype: str, cuts_for, block_size: int = 16) -> np.ndarray:
    """Decode attention computed per context partition and merged.

    `cuts_for(s, ctx)` returns the interior cut points of sequence s. The
    result equals decode_attention up to float64 rounding for any cuts.
    """
    q = widen(q, dtype)
    S, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    out = np.zeros((S, Hq, D))
    for s in range(S):
        ctx = int(context_lens[s])
        if ctx == 0:
            continue
        Kc = widen(gather_sequence(k_pool, block_tables[s], ctx, block_size), dtype)
        Vc = widen(gather_sequence(v_pool, block_tables[s], ctx, block_size), dtype)
        bounds = [0] + sorted(int(c) for c in cuts_for(s, ctx)) + [ctx]
        for hq in range(Hq):
            h = _kv_head(hq, Hq, Hkv)
            parts = [partial_attention(Kc[a:b, h], Vc[a:b, h], q[s, hq], scale)
                     for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
            out[s, hq] = merge_partials(parts)
    return out


def _bits(a: np.ndarray) -> np.ndarray:
    """View any 1-, 2- or 4-byte array as unsigned integers (raw bit copies;
    1-byte elements are the codes of an fp8 cache)."""
    return a.view({1: np.uint8, 2: np.uint16, 4: np.uint32}[a.dtype.itemsize])


def reshape_and_cache(k_new, v_new, k_pool, v_pool, slots, block_size: int = 16) -> None:
    """Write each new token's K and V into its slot, in place, as raw bits.

    [3] ("The allocation lifecycle") writes each decode step's K,V into the
    sequence's last block; the slot comes from the slot formula of [4].
    k_new/v_new are [T, Hkv, D]; slots < 0 are skipped.
    """
    kp, vp = _bits(k_pool), _bits(v_pool)
    kn, vn = _bits(np.ascontiguousarray(k_new)), _bits(np.ascontiguousarray(v_new))
    for i, s in enumerate(np.asarray(slots, dtype=np.int64)):
        s = int(s)
        if s < 0:
            continue
        kp[s // block_size, :, s % block_size, :] = kn[i]
        vp[s // block_size, :, s % block_size, :] = vn[i]


def copy_blocks(pools: List[np.ndarray], pairs: Sequence[Tuple[int, int]]) -> None:
    """Copy whole physical blocks src -> dst in every given pool, in place.

    This is the device half of copy-on-write ([2], "Copy-on-Write for Beam
    Search and Parallel Sampling"): the manager allocates a block and copies
    the shared block's content into it. Pairs are applied in order.
    """
    for pool in pools:
        b = _bits(pool)
        for src, dst in pairs:
            b[int(dst)] = b[int(src)]


def swap_out_blocks(k_pools: List[np.ndarray], v_pools: List[np.ndarray],
                    ids: Sequence[int]) -> np.ndarray:
    """Host copy of whole blocks for a swap-out, as raw bytes laid out
    [n][layer][K, V][block bytes] (one block's state for all layers together).

    The device half of preemption by swapping ([3], "The allocation
    lifecycle", memory pressure; [1], "Preemption"): the block contents move
    to host memory unchanged. Entries outside the pool are left as zeros.
    """
    L = len(k_pools)
    nb = k_pools[0].shape[0]
    bb = k_pools[0][0].nbytes
    host = np.zeros((len(ids), L, 2, bb), dtype=np.uint8)
    for i, b in enumerate(ids):
        if not (0 <= int(b) < nb):
            continue
        for layer in range(L):
            host[i, layer, 0] = np.frombuffer(np.ascontiguousarray(k_pools[layer][int(b)]).tobytes(),
                                              dtype=np.uint8)
            host[i, layer, 1] = np.frombuffer(np.ascontiguousarray(v_pools[layer][int(b)]).tobytes(),
                                              dtype=np.uint8)
    return host


def swap_in_blocks(k_pools: List[np.ndarray], v_pools: List[np.ndarray],
                   ids: Sequence[int], host: np.ndarray) -> None:
    """Inverse of swap_out_blocks: write host[i] back into block ids[i] of
    every layer, in place (entries outside the pool are skipped)."""
    nb = k_pools[0].shape[0]
    for i, b in enumerate(ids):
        if not (0 <= int(b) < nb):
            continue
        for layer, (kp, vp) in enumerate(zip(k_pools, v_pools)):
            for pool, kv in ((kp, 0), (vp, 1)):
                blk = pool[int(b)]
                pool[int(b)] = np.frombuffer(host[i, layer, kv].tobytes(),
                                             dtype=pool.dtype).reshape(blk.shape)


def prefill_attention(q, q_start, k_pool, v_pool, block_tables, context_lens, scale: float,
                      dtype: str, block_size: int = 16,
                      rows: Optional[Iterable[int]] = None, kv_dtype: Optional[str] = None,
                      k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Attention of a chunk of new query tokens per sequence over the paged
    cache, causal within the chunk. Chunked prefill processes a prompt in
    pieces of a fixed token count ([2] "The Successors - SGLang's
    RadixAttention and Prefix Sharing"); the chunk's K/V are written into the
    sequence's blocks first ([2] "Walking Through the Lifecycle", Prefill).

    q is packed [T, Hq, D]; the tokens of sequence s are rows
    q_start[s] .. q_start[s+1]-1, C_s of them, and context_lens[s] = L_s counts
    every cached position of s including the chunk's own (already written).
    Query row i of the chunk sits at position p = L_s - C_s + i and attends to
    positions 0..p: out = sum_j w_j V[j] / sum_j w_j, w_j = exp(z_j - max z),
    z_j = scale * <q, K[j]>. Returns float64 [T, Hq, D]; with `rows`, only
    those query rows are computed and the rest stay NaN. `kv_dtype` and the
    scales describe an fp8 cache as in decode_attention.
    """
    q = widen(q, dtype)
    T, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    out = np.full((T, Hq, D), np.nan)
    want = None if rows is None else set(int(r) for r in rows)
    sc = float(np.float64(scale))
    S = len(q_start) - 1
    for s in range(S):
        r0, r1 = int(q_start[s]), int(q_start[s + 1])
        if r1 <= r0 or (want is not None and not any(r0 <= r < r1 for r in want)):
            continue
        L = int(context_lens[s])
        C = r1 - r0
        if C > L:
            raise ValueError(f"sequence {s}: chunk of {C} tokens longer than its context {L}")
        kd = kv_dtype or dtype
        Kc = widen(gather_sequence(k_pool, block_tables[s], L, block_size), kd)
        Vc = widen(gather_sequence(v_pool, block_tables[s], L, block_size), kd)
        if kv_dtype is not None:
            Kc = Kc * float(np.float32(k_scale))
            Vc = Vc * float(np.float32(v_scale))
        for i in range(C):
            r = r0 + i
            if want is not None and r not in want:
                continue
            p = L - C + i
            for hq in range(Hq):
                h = _kv_head(hq, Hq, Hkv)
                z = sc * (Kc[:p + 1, h, :] @ q[r, hq])
                w = np.exp(z - z.max())
                out[r, hq] = (w @ Vc[:p + 1, h, :]) / w.sum()
    return out
