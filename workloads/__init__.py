"""Seeded synthetic inputs for the paged decode-attention workloads.

This module only draws random numbers and describes workload shapes and
operation scripts. It holds none of the method's arithmetic: no slot
formula, no block-table construction, no attention. Both the CPU oracle and
the GPU library consume what it produces, each with its own code.

Pages cited in this file:
  [1] "PagedAttention - how vLLM stopped wasting 80% of your GPU memory"
      (shivam2003.com/posts/pagedattention.html)
  [2] "PagedAttention: How vLLM Borrowed Virtual Memory to Unlock GPU Serving
      at Scale" (fp4-site.pages.dev/system/pagedattention-vllm-deep-dive/)
  [3] "PagedAttention and vLLM: Virtual Memory for the KV Cache"
      (passgenai.com, lesson 12-07 of the NCA-GENL course)

Workload recipe (all seeded):
  * context lengths per the workload spec; lengths include the token decoded
    in the current step;
  * a permutation of all physical block IDs: the order in which the block
    manager hands blocks out (the pool is "shuffled");
  * every slot of both pools is N(0,1) in fp32, rounded to the storage dtype
    with round-to-nearest-even; unused slots therefore hold finite data unless
    a test poisons them;
  * the query and the new token's K/V are N(0,1), rounded the same way;
  * an fp8 cache (workload 7) holds random E4M3 codes instead: each byte has
    a uniform sign bit, an exponent field uniform in 0..9 (field 0 gives the
    subnormals and zero) and a uniform mantissa, i.e. magnitudes up to 7.5,
    read with a per-pool scale of 1/4; the new token's K/V stay 16-bit
    N(0,1) values (the cache write quantises them);
  * an operation script (create / append / fork) that builds the sequences;
  * the chunked-prefill workload (8) gives every sequence a cached prefix
    (lognormal like workload 3) and a chunk of new tokens: its queries are
    [S * chunk, Hq, D] and its new K/V [S * chunk, Hkv, D], N(0,1) as above.
Heavy-tailed lengths follow the shape [2] describes for production traffic
("The Fragmentation Problem"): many short requests and a long tail. The
lognormal spread is taken from the eight-request sample of [3] ("A
constructed scenario"), whose log-lengths have a sample standard deviation
of about 0.86.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Tuple

import numpy as np

__all__ = [
    "WorkloadSpec", "Workload", "SPECS", "spec", "make_workload",
    "round_to_dtype", "bf16_bits_to_f32", "NP_STORAGE",
]

# Storage dtypes. bf16 is held as raw uint16 bit patterns on the host side
# because numpy has no bfloat16 type.
NP_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "e4m3": np.uint8}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to the storage dtype with round-to-nearest-even.

    bf16 results are returned as uint16 bit patterns (upper half of the fp32
    encoding after rounding). NaN stays a quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        lsb = (u >> 16) & 1
        r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
        nan = np.isnan(x)
        if nan.any():
            r[nan] = 0x7FC0
        return r
    raise ValueError(f"unknown dtype {dtype!r}")


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 (used for printing/plots)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    cfg: int                 # 1..5, 6 = the copy-on-write variant of 5
    name: str
    S: int                   # sequences
    Hq: int                  # query heads
    Hkv: int                 # KV heads
    D: int                   # head_dim
    dtype: str               # "f32" | "f16" | "bf16"
    block_size: int = 16
    partition_size: int = 512
    # prefix sharing (cfg 5/6): tokens shared by all sequences, and tail
    # tokens each sequence appends after the fork
    shared_prefix: int = 0
    tail: int = 0
    # cache storage when it differs from `dtype` (the query's type): "e4m3",
    # with one scale per pool
    kv_dtype: str = ""
    k_scale: float = 1.0
    v_scale: float = 1.0
    # default seed taken from this workload number (same lengths and queries)
    seed_cfg: int = 0
    # chunked prefill: query tokens per sequence in the step (0 = decode, 1 token)
    chunk: int = 0
    description: str = ""

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        # fp32-rounded 1/sqrt(head_dim); both sides use this same value
        return float(np.float32(1.0 / math.sqrt(self.D)))

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]

    @property
    def cache_dtype(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def kv_elem_bytes(self) -> int:
        return ELEM_BYTES[self.cache_dtype]


SPECS = {
    1: WorkloadSpec(1, "tiny-fp32", S=4, Hq=4, Hkv=4, D=64, dtype="f32",
                    description="4 sequences, lengths {5,16,17,40}, 4 heads, "
                                "head_dim 64, fp32, pool of 32 blocks"),
    2: WorkloadSpec(2, "llama13b-mha-fp16", S=64, Hq=40, Hkv=40, D=128, dtype="f16",
                    description="64 sequences, lengths uniform in [128,2048], "
                                "40 heads, head_dim 128, fp16, 8192-block pool"),
    3: WorkloadSpec(3, "llama70b-gqa-bf16", S=128, Hq=64, Hkv=8, D=128, dtype="bf16",
                    description="128 sequences, lognormal lengths (median 512, "
                                "sigma 0.86, clipped to [16,8192]), 64 query / "
                                "8 KV heads, head_dim 128, bf16"),
    4: WorkloadSpec(4, "longctx-splitk-bf16", S=8, Hq=32, Hkv=8, D=128, dtype="bf16",
                    description="8 sequences at 32768 tokens, 32 query / 8 KV "
                                "heads, head_dim 128, bf16, 512-token partitions"),
    5: WorkloadSpec(5, "prefix-share-bf16", S=32, Hq=32, Hkv=8, D=128, dtype="bf16",
                    shared_prefix=2048, tail=256,
                    description="32 sequences sharing a 2048-token prefix, 256 "
                                "own tail tokens each, one decode token; 32 "
                                "query / 8 KV heads, head_dim 128, bf16"),
    6: WorkloadSpec(6, "prefix-cow-bf16", S=32, Hq=32, Hkv=8, D=128, dtype="bf16",
                    shared_prefix=2056, tail=248,
                    description="as the prefix-share workload but forked inside "
                                "a block (2056 shared tokens), so the first "
                                "write of each fork copies the partial block"),
    8: WorkloadSpec(8, "llama70b-gqa-chunked-prefill-bf16", S=16, Hq=64, Hkv=8, D=128,
                    dtype="bf16", chunk=256,
                    description="16 sequences, each with a cached prefix of "
                                "lognormal length (median 512, sigma 0.86) and "
                                "a 256-token chunk attended causally; 64 query / "
                                "8 KV heads, head_dim 128, bf16"),
    9: WorkloadSpec(9, "llama70b-gqa-chunked-prefill-fp8", S=16, Hq=64, Hkv=8, D=128,
                    dtype="bf16", chunk=256, kv_dtype="e4m3", k_scale=0.25, v_scale=0.25,
                    seed_cfg=8,
                    description="the chunked-prefill workload (same prefixes, chunks "
                                "and queries) over an fp8 E4M3 cache with per-pool "
                                "scales"),
    10: WorkloadSpec(10, "llama70b-gqa-longprefix-prefill-bf16", S=4, Hq=64, Hkv=8, D=128,
                     dtype="bf16", chunk=16,
                     description="4 sequences, each with a 32752-token cached prefix "
                                 "and a 16-token chunk attended causally (context "
                                 "32768); 64 query / 8 KV heads, head_dim 128, bf16"),
    11: WorkloadSpec(11, "prefix-share-long-fp8", S=64, Hq=32, Hkv=8, D=128, dtype="bf16",
                     kv_dtype="e4m3", k_scale=0.25, v_scale=0.25, shared_prefix=4096, tail=256,
                     description="64 sequences sharing a 4096-token prefix, 256 own tail "
                                 "tokens each, one decode token; 32 query / 8 KV heads, "
                                 "head_dim 128, bf16 queries over an fp8 E4M3 cache with "
                                 "per-pool scales"),
    7: WorkloadSpec(7, "llama70b-gqa-fp8", S=128, Hq=64, Hkv=8, D=128, dtype="bf16",
                    kv_dtype="e4m3", k_scale=0.25, v_scale=0.25, seed_cfg=3,
                    description="the llama70b-gqa-bf16 workload (same lengths, "
                                "queries and new tokens) over an fp8 E4M3 "
                                "cache with per-pool scales"),
}


def spec(cfg: int) -> WorkloadSpec:
    return SPECS[cfg]


# Operation script entries: ("create", seq) | ("append", seq, n) |
# ("append", seq, n, "values") | ("fork", parent, child). Sequence handles are
# small integers local to the script; each side maps them to its own handles.
# An append tagged "values" writes the sequence's next rows of tail_k/tail_v
# into the new slots; untagged appends reserve slots whose content is the
# pool's synthetic fill.
Op = Tuple


@dataclasses.dataclass
class Workload:
    spec: WorkloadSpec
    context_lens: np.ndarray          # int32 [S], including the decode token
    num_blocks: int
    free_order: np.ndarray            # int32 [num_blocks], first handed out first
    setup_ops: List[Op]               # builds every sequence up to ctx-1 tokens
    step_ops: List[Op]                # the decode step: append 1 token per sequence
    q: np.ndarray                     # [S, Hq, D] storage dtype
    k_pool: np.ndarray                # [NB, Hkv, B, D] storage dtype
    v_pool: np.ndarray
    k_new: np.ndarray                 # [S, Hkv, D] the decode token's K
    v_new: np.ndarray
    tail_k: Optional[np.ndarray] = None   # [S, tail, Hkv, D] (cfg 5/6)
    tail_v: Optional[np.ndarray] = None

    @property
    def S(self):
        return self.spec.S


def _normal(rng: np.random.Generator, shape, dtype: str, chunk=1 << 26) -> np.ndarray:
    """N(0,1) fp32 draws rounded to the storage dtype, generated in chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=NP_STORAGE[dtype])
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = round_to_dtype(rng.standard_normal(e - s, dtype=np.float32), dtype)
    return out.reshape(shape)


def _e4m3_codes(rng: np.random.Generator, shape, chunk=1 << 26) -> np.ndarray:
    """Random E4M3 bytes: uniform sign, exponent field uniform in 0..9,
    uniform mantissa (no NaN code can occur)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint8)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        sign = rng.integers(0, 2, e - s, dtype=np.uint8)
        expo = rng.integers(0, 10, e - s, dtype=np.uint8)
        mant = rng.integers(0, 8, e - s, dtype=np.uint8)
        out[s:e] = (sign << 7) | (expo << 3) | mant
    return out.reshape(shape)


def _context_lengths(sp: WorkloadSpec, rng: np.random.Generator) -> np.ndarray:
    if sp.cfg == 1:
        return np.array([5, 16, 17, 40], dtype=np.int32)
    if sp.cfg == 2:
        return rng.integers(128, 2048, size=sp.S, endpoint=True).astype(np.int32)
    if sp.cfg in (3, 7):
        x = np.exp(rng.normal(math.log(512.0), 0.86, size=sp.S))
        return np.clip(np.rint(x), 16, 8192).astype(np.int32)
    if sp.cfg in (8, 9):
        x = np.exp(rng.normal(math.log(512.0), 0.86, size=sp.S))
        return (np.clip(np.rint(x), 0, 8192 - sp.chunk) + sp.chunk).astype(np.int32)
    if sp.cfg in (4, 10):
        return np.full(sp.S, 32768, dtype=np.int32)
    if sp.cfg in (5, 6, 11):
        return np.full(sp.S, sp.shared_prefix + sp.tail + 1, dtype=np.int32)
    raise ValueError(sp.cfg)


def _pool_blocks(sp: WorkloadSpec, lens: np.ndarray) -> int:
    """Pool size per the workload spec (an input, not the allocator's answer)."""
    B = sp.block_size
    if sp.cfg == 1:
        return 32
    if sp.cfg == 2:
        return 8192 * 16 // B  # the worst case, 64 sequences of 2048 tokens
    if sp.cfg in (3, 7, 8, 9, 10):
        need = int(sum(-(-int(t) // B) for t in lens))
        return int(math.ceil(1.1 * need))
    if sp.cfg == 4:
        return int(sp.S * (32768 // B))
    if sp.cfg in (5, 6, 11):
        # shared prefix once plus every sequence's own blocks, +10%
        pre = -(-sp.shared_prefix // B)
        own = -(-(sp.shared_prefix + sp.tail + 1) // B) - sp.shared_prefix // B
        return int(math.ceil(1.1 * (pre + sp.S * own)))
    raise ValueError(sp.cfg)


def make_workload(cfg: int, seed: Optional[int] = None, *, with_values: bool = True,
                  S: Optional[int] = None, block_size: int = 16) -> Workload:
    """Build workload `cfg` deterministically.

    `seed` defaults to 162000 + cfg. `with_values=False` skips the pool fill
    (for host-only allocator tests). `S` optionally truncates the number of
    sequences of the randomly-sized workloads (2 and 3) for small CPU tests;
    the pool is then sized for that S with the same rule.
    """
    sp = SPECS[cfg]
    if block_size != sp.block_size:
        # the same workload in another block size: same lengths, queries and
        # new tokens; the pool is sized by the same rule for the new block size
        sp = dataclasses.replace(sp, block_size=block_size)
    if S is not None and S != sp.S:
        if cfg not in (2, 3, 4, 7):
            raise ValueError("only workloads 2-4 and 7 may be truncated")
        sp = dataclasses.replace(sp, S=S)
    ss = np.random.SeedSequence(162_000 + (sp.seed_cfg or cfg) if seed is None else seed)
    r_len, r_perm, r_q, r_k, r_v, r_new = [np.random.default_rng(s) for s in ss.spawn(6)]

    lens = _context_lengths(sp, r_len)
    if S is not None:
        lens = lens[:S]
    NB = _pool_blocks(sp, lens)
    free_order = r_perm.permutation(NB).astype(np.int32)

    setup: List[Op] = []
    step: List[Op] = []
    if sp.shared_prefix:
        setup.append(("create", 0))
        setup.append(("append", 0, sp.shared_prefix))
        for c in range(1, sp.S):
            setup.append(("fork", 0, c))
        for s_ in range(sp.S):
            # tagged: these tokens' K/V are written from tail_k / tail_v
            setup.append(("append", s_, sp.tail, "values"))
    else:
        step_n = sp.chunk or 1
        for s_ in range(sp.S):
            setup.append(("create", s_))
            if int(lens[s_]) > step_n:
                setup.append(("append", s_, int(lens[s_]) - step_n))
    for s_ in range(sp.S):
        step.append(("append", s_, sp.chunk or 1))

    Hkv, D, B = sp.Hkv, sp.D, sp.block_size
    if with_values:
        T = sp.S * (sp.chunk or 1)
        q = _normal(r_q, (T, sp.Hq, D), sp.dtype) if sp.chunk else _normal(r_q, (sp.S, sp.Hq, D), sp.dtype)
        if sp.kv_dtype == "e4m3":
            k_pool = _e4m3_codes(r_k, (NB, Hkv, B, D))
            v_pool = _e4m3_codes(r_v, (NB, Hkv, B, D))
        else:
            k_pool = _normal(r_k, (NB, Hkv, B, D), sp.dtype)
            v_pool = _normal(r_v, (NB, Hkv, B, D), sp.dtype)
        k_new = _normal(r_new, (T, Hkv, D), sp.dtype)
        v_new = _normal(r_new, (T, Hkv, D), sp.dtype)
        tail_k = tail_v = None
        if sp.shared_prefix:
            tail_k = _normal(r_new, (sp.S, sp.tail, Hkv, D), sp.dtype)
            tail_v = _normal(r_new, (sp.S, sp.tail, Hkv, D), sp.dtype)
    else:
        z = np.zeros(0, dtype=NP_STORAGE[sp.dtype])
        q = k_new = v_new = z
        k_pool = v_pool = np.zeros(0, dtype=NP_STORAGE[sp.cache_dtype])
        tail_k = tail_v = None
    return Workload(spec=sp, context_lens=lens.astype(np.int32), num_blocks=NB,
                    free_order=free_order, setup_ops=setup, step_ops=step,
                    q=q, k_pool=k_pool, v_pool=v_pool, k_new=k_new, v_new=v_new,
                    tail_k=tail_k, tail_v=tail_v)
