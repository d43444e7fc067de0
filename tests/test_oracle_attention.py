"""Pins for the attention oracle (CPU only).

Each test ties oracle/attention.py to something other than itself: brute
force on unpaged arrays, a library routine, closed-form special cases,
invariants the pages state, and planted mistakes that the pins must catch.

Pages cited:
  [1] "PagedAttention - how vLLM stopped wasting 80% of your GPU memory"
      (shivam2003.com/posts/pagedattention.html)
  [2] "PagedAttention: How vLLM Borrowed Virtual Memory to Unlock GPU Serving
      at Scale" (fp4-site.pages.dev/system/pagedattention-vllm-deep-dive/)
  [3] "PagedAttention and vLLM: Virtual Memory for the KV Cache" (passgenai.com)
  [4] "What is paged attention?" (netraruntime.com/learn/paged-attention)
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oa
from workloads import round_to_dtype, make_workload

B = 16


# ---------------------------------------------------------------------------
# helpers written independently of the oracle
# ---------------------------------------------------------------------------
def place_contiguous(seqs_k, seqs_v, tables, num_blocks, Hkv, D, fill=np.nan, dtype=np.float64):
    """Place each sequence's contiguous cache into a pool by walking its block
    table: entry i of a sequence's table holds tokens i*B .. i*B+B-1 ([2],
    "The OS-Inspired Insight", item 2). Unused slots get `fill`."""
    kp = np.full((num_blocks, Hkv, B, D), fill, dtype=dtype)
    vp = np.full((num_blocks, Hkv, B, D), fill, dtype=dtype)
    for Kc, Vc, table in zip(seqs_k, seqs_v, tables):
        for i, phys in enumerate(table):
            if phys < 0:
                continue
            for j in range(B):
                tok = i * B + j
                if tok < len(Kc):
                    kp[phys, :, j, :] = Kc[tok]
                    vp[phys, :, j, :] = Vc[tok]
    return kp, vp


def brute_force(q, seqs_k, seqs_v, scale):
    """Softmax attention with plain Python loops over unpaged arrays."""
    S, Hq, D = q.shape
    out = np.zeros((S, Hq, D))
    for s in range(S):
        Kc, Vc = seqs_k[s], seqs_v[s]
        t = len(Kc)
        Hkv = Kc.shape[1] if t else 1
        G = Hq // Hkv
        for hq in range(Hq):
            h = hq // G
            z = []
            for j in range(t):
                acc = 0.0
                for d in range(D):
                    acc += float(q[s, hq, d]) * float(Kc[j, h, d])
                z.append(scale * acc)
            if not z:
                continue
            zm = max(z)
            w = [math.exp(x - zm) for x in z]
            tot = sum(w)
            for d in range(D):
                out[s, hq, d] = sum(w[j] * float(Vc[j, h, d]) for j in range(t)) / tot
    return out


def random_paged_case(rng, lens, Hq, Hkv, D, num_blocks=None):
    seqs_k = [rng.standard_normal((t, Hkv, D)) for t in lens]
    seqs_v = [rng.standard_normal((t, Hkv, D)) for t in lens]
    nbs = [-(-t // B) for t in lens]
    if num_blocks is None:
        num_blocks = sum(nbs) + 3
    perm = rng.permutation(num_blocks)
    tables, off = [], 0
    maxb = max(nbs + [1])
    tab = np.full((len(lens), maxb), -1, dtype=np.int32)
    for s, nb in enumerate(nbs):
        tab[s, :nb] = perm[off:off + nb]
        tables.append(list(perm[off:off + nb]))
        off += nb
    kp, vp = place_contiguous(seqs_k, seqs_v, tables, num_blocks, Hkv, D)
    q = rng.standard_normal((len(lens), Hq, D))
    return q, kp, vp, tab, np.array(lens, dtype=np.int32), seqs_k, seqs_v


# ---------------------------------------------------------------------------
# storage widening and input rounding
# ---------------------------------------------------------------------------
def test_widen_bf16_known_bits():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F80, 0x0001], dtype=np.uint16)
    w = oa.widen(bits, "bf16")
    assert w[0] == 1.0 and w[1] == -2.0 and w[2] == 1.0 + 2.0 ** -7
    assert w[3] == 0.0 and math.copysign(1, w[4]) == -1.0 and w[5] == math.inf
    assert w[6] == 2.0 ** -133  # smallest bf16 subnormal


def test_round_to_bf16_matches_torch_and_ties_to_even():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(100_000).astype(np.float32) * 10
    ours = round_to_dtype(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # exact halfway cases round to the even neighbour
    half = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], dtype=np.float32)
    assert list(round_to_dtype(half, "bf16")) == [0x3F80, 0x3F82]


def test_round_to_f16_is_ieee():
    x = np.array([1.0 + 2.0 ** -11, 65504.0, 1e-8], dtype=np.float32)
    r = round_to_dtype(x, "f16")
    assert r[0] == np.float16(1.0) and r[1] == np.float16(65504.0)


# ---------------------------------------------------------------------------
# slot formula, scatter, copy
# ---------------------------------------------------------------------------
def test_slot_formula_closed_form():
    # [4], "How it works": slot(p) = table[floor(p/16)] * 16 + p mod 16
    table = [7, 3, 11]
    assert [oa.slot_of(table, p) for p in (0, 15, 16, 31, 32, 39)] == [112, 127, 48, 63, 176, 183]


def test_slot_mapping_invalid_entries():
    tables = np.array([[5, 2, -1], [0, 1, 4]], dtype=np.int32)
    seq = np.array([0, 0, 0, 1, 1, 0])
    pos = np.array([17, 40, -1, 47, 48, 0])
    got = oa.slot_mapping(tables, seq, pos)
    assert list(got) == [2 * 16 + 1, -1, -1, 4 * 16 + 15, -1, 5 * 16]


def test_slot_roundtrip_scatter_then_blockwalk():
    """Scatter contiguous rows by slot, read them back by walking whole
    physical blocks in table order: identity on every live position."""
    rng = np.random.default_rng(3)
    lens = [1, 15, 16, 17, 40, 33]
    nbs = [-(-t // B) for t in lens]
    perm = rng.permutation(sum(nbs))
    tabs, off = [], 0
    for nb in nbs:
        tabs.append(list(perm[off:off + nb]))
        off += nb
    pool = np.full((sum(nbs), 1, B, 1), np.nan)
    for s, t in enumerate(lens):
        for p in range(t):
            sl = oa.slot_of(tabs[s], p)
            pool[sl // B, 0, sl % B, 0] = 1000 * s + p
    for s, t in enumerate(lens):
        walk = np.concatenate([pool[b, 0, :, 0] for b in tabs[s]])[:t]
        assert list(walk) == [1000 * s + p for p in range(t)]
    # unshared live (seq, p) pairs map to distinct slots
    allslots = [oa.slot_of(tabs[s], p) for s, t in enumerate(lens) for p in range(t)]
    assert len(set(allslots)) == len(allslots)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_reshape_and_cache_is_a_raw_bit_copy(dtype):
    rng = np.random.default_rng(4)
    NB, Hkv, D = 5, 2, 8
    store = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]
    kp = np.zeros((NB, Hkv, B, D), dtype=store)
    vp = np.zeros((NB, Hkv, B, D), dtype=store)
    nbytes = np.dtype(store).itemsize
    ut = {2: np.uint16, 4: np.uint32}[nbytes]
    kn = rng.integers(0, 2 ** (8 * nbytes), size=(3, Hkv, D), dtype=np.uint64).astype(ut)
    vn = rng.integers(0, 2 ** (8 * nbytes), size=(3, Hkv, D), dtype=np.uint64).astype(ut)
    # include NaN payloads and negative zero bit patterns
    kn[0, 0, 0] = 0x7FC1 if nbytes == 2 else 0x7FC00001
    kn[0, 0, 1] = 0x8000 if nbytes == 2 else 0x80000000
    slots = np.array([3 * 16 + 5, -1, 0 * 16 + 15])
    oa.reshape_and_cache(kn.view(store), vn.view(store), kp, vp, slots)
    assert np.array_equal(kp.view(ut)[3, :, 5, :], kn[0])
    assert np.array_equal(vp.view(ut)[3, :, 5, :], vn[0])
    assert np.array_equal(kp.view(ut)[0, :, 15, :], kn[2])
    written = np.zeros((NB, B), bool)
    written[3, 5] = written[0, 15] = True
    assert not kp.view(ut).transpose(0, 2, 1, 3)[~written].any()  # nothing else written


def test_copy_blocks_bits():
    a = np.arange(4 * 2 * B * 3, dtype=np.uint16).reshape(4, 2, B, 3)
    b = a.copy() + 1
    oa.copy_blocks([a, b], [(0, 3), (1, 2)])
    assert np.array_equal(a[3], a[0]) and np.array_equal(a[2], a[1])
    assert np.array_equal(b[3], b[0]) and np.array_equal(b[2], b[1])


def test_copy_blocks_fp8_codes():
    """A block of an fp8 cache is copied byte for byte, NaN codes included; the
    other blocks are untouched."""
    rng = np.random.default_rng(3)
    a = rng.integers(0, 256, (5, 2, B, 8), dtype=np.uint8)
    a[1, 0, 0, 0] = 0x7F                      # an E4M3 NaN code travels as a byte
    before = a.copy()
    oa.copy_blocks([a], [(1, 4), (0, 2)])
    assert np.array_equal(a[4], before[1]) and np.array_equal(a[2], before[0])
    assert a[4, 0, 0, 0] == 0x7F
    assert np.array_equal(a[[0, 1, 3]], before[[0, 1, 3]])


# ---------------------------------------------------------------------------
# attention: brute force and a library routine
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (8, 1)])
def test_oracle_matches_brute_force_on_unpaged_arrays(Hq, Hkv):
    rng = np.random.default_rng(10 + Hq + Hkv)
    lens = [5, 16, 17, 40, 1]
    D = 8
    q, kp, vp, tab, cl, sk, sv = random_paged_case(rng, lens, Hq, Hkv, D)
    scale = 1 / math.sqrt(D)
    got = oracle.decode_attention(q.astype(np.float32), kp.astype(np.float32),
                                  vp.astype(np.float32), tab, cl, scale, "f32")
    # brute force sees the same fp32-rounded inputs
    q32 = q.astype(np.float32).astype(np.float64)
    sk32 = [k.astype(np.float32).astype(np.float64) for k in sk]
    sv32 = [v.astype(np.float32).astype(np.float64) for v in sv]
    ref = brute_force(q32, sk32, sv32, scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_oracle_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(11)
    lens = [7, 33, 64, 100]
    Hq, Hkv, D = 8, 2, 32
    q, kp, vp, tab, cl, sk, sv = random_paged_case(rng, lens, Hq, Hkv, D)
    scale = 0.17
    got = oracle.decode_attention(q, kp, vp, tab, cl, scale, "f32")
    for s, t in enumerate(lens):
        K = torch.from_numpy(np.repeat(sk[s], Hq // Hkv, axis=1)).permute(1, 0, 2)  # [Hq,t,D]
        V = torch.from_numpy(np.repeat(sv[s], Hq // Hkv, axis=1)).permute(1, 0, 2)
        Q = torch.from_numpy(q[s]).unsqueeze(1)                                   # [Hq,1,D]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)
        np.testing.assert_allclose(got[s], ref[:, 0].numpy(), rtol=0, atol=1e-12)


def test_second_loop_order_agrees_on_the_tiny_workload_with_poisoned_slots():
    w = make_workload(1)
    bm = oracle.BlockManager(w.num_blocks, free_order=w.free_order)
    from oracle.block_manager import run_ops
    h, _, _ = run_ops(bm, w.setup_ops + w.step_ops)
    seqs = [h[i] for i in range(w.S)]
    tab, cl = bm.packed_tables(seqs)
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    # poison every slot no sequence uses
    live = np.zeros((w.num_blocks, B), bool)
    for s, t in enumerate(cl):
        for p in range(t):
            sl = oa.slot_of(tab[s], p)
            live[sl // B, sl % B] = True
    dead = ~live[:, None, :]                       # broadcast over KV heads
    kp[np.broadcast_to(dead, kp.shape[:3])] = np.nan
    vp[np.broadcast_to(dead, vp.shape[:3])] = np.nan
    a = oracle.decode_attention(w.q, kp, vp, tab, cl, w.spec.scale, "f32")
    b = oracle.decode_attention_blockwise(w.q, kp, vp, tab, cl, w.spec.scale, "f32")
    assert np.isfinite(a).all()
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# closed-form special cases
# ---------------------------------------------------------------------------
def _one(lens, Hq=2, Hkv=1, D=4, seed=0):
    rng = np.random.default_rng(seed)
    return random_paged_case(rng, lens, Hq, Hkv, D)


def test_single_token_returns_its_value_exactly():
    q, kp, vp, tab, cl, sk, sv = _one([1])
    out = oracle.decode_attention(q, kp, vp, tab, cl, 0.5, "f32")
    assert np.array_equal(out[0, 0], sv[0][0, 0]) and np.array_equal(out[0, 1], sv[0][0, 0])


def test_equal_values_return_that_value():
    q, kp, vp, tab, cl, sk, sv = _one([37])
    v = np.array([0.25, -1.5, 3.0, 0.125])
    vp[np.isfinite(vp[..., 0])] = v
    out = oracle.decode_attention(q, kp, vp, tab, cl, 0.5, "f32")
    np.testing.assert_allclose(out[0], np.tile(v, (2, 1)), rtol=0, atol=1e-15)


@pytest.mark.parametrize("zero", ["scale", "query"])
def test_zero_scores_give_the_mean_of_values(zero):
    q, kp, vp, tab, cl, sk, sv = _one([29])
    scale = 0.0 if zero == "scale" else 0.7
    if zero == "query":
        q[:] = 0
    out = oracle.decode_attention(q, kp, vp, tab, cl, scale, "f32")
    np.testing.assert_allclose(out[0, 0], sv[0][:, 0].mean(axis=0), rtol=0, atol=1e-14)


def test_one_dominant_key_selects_its_value():
    q, kp, vp, tab, cl, sk, sv = _one([21], Hq=1)
    j = 13
    q[0, 0] = 50 * sk[0][j, 0] / np.linalg.norm(sk[0][j, 0])
    # make key j clearly dominant
    kp_ = kp.copy()
    slot = oa.slot_of(tab[0], j)
    kp_[slot // B, 0, slot % B] = 10 * q[0, 0] / np.linalg.norm(q[0, 0])
    out = oracle.decode_attention(q, kp_, vp, tab, cl, 1.0, "f32")
    np.testing.assert_allclose(out[0, 0], sv[0][j, 0], rtol=0, atol=1e-12)


def test_empty_sequence_gives_zero():
    q, kp, vp, tab, cl, sk, sv = _one([9])
    cl2 = np.array([0], dtype=np.int32)
    out = oracle.decode_attention(q, kp, vp, tab, cl2, 1.0, "f32")
    assert np.array_equal(out, np.zeros_like(out))


# ---------------------------------------------------------------------------
# invariants the pages state
# ---------------------------------------------------------------------------
def test_placement_invariance_bitwise():
    """[1] ("FAQ": outputs do not change) and [3] ("The kernel change"): the
    same cache stored contiguously or in shuffled blocks gives the same
    attention - bit for bit in the oracle, since it gathers by position."""
    rng = np.random.default_rng(21)
    lens = [3, 16, 50, 77]
    Hq, Hkv, D = 4, 2, 16
    sk = [rng.standard_normal((t, Hkv, D)) for t in lens]
    sv = [rng.standard_normal((t, Hkv, D)) for t in lens]
    q = rng.standard_normal((len(lens), Hq, D))
    nbs = [-(-t // B) for t in lens]
    NB = sum(nbs)
    outs = []
    for order in (np.arange(NB), rng.permutation(NB), rng.permutation(NB)):
        tabs, off = [], 0
        tab = np.full((len(lens), max(nbs)), -1, np.int32)
        for s, nb in enumerate(nbs):
            tabs.append(list(order[off:off + nb]))
            tab[s, :nb] = order[off:off + nb]
            off += nb
        kp, vp = place_contiguous(sk, sv, tabs, NB, Hkv, D)
        outs.append(oracle.decode_attention(q, kp, vp, tab, np.array(lens), 0.3, "f32"))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_shared_prefix_equals_duplicated_prefix_bitwise():
    """[3] ("Copy-on-write sharing"): a shared prefix holds the same K and V
    for every sequence, so sharing its blocks equals storing copies."""
    rng = np.random.default_rng(22)
    Hq, Hkv, D, pre, tails = 4, 1, 8, 48, [5, 17, 30]
    pk = rng.standard_normal((pre, Hkv, D))
    pv = rng.standard_normal((pre, Hkv, D))
    sk = [np.concatenate([pk, rng.standard_normal((t, Hkv, D))]) for t in tails]
    sv = [np.concatenate([pv, rng.standard_normal((t, Hkv, D))]) for t in tails]
    q = rng.standard_normal((len(tails), Hq, D))
    lens = np.array([pre + t for t in tails])
    # unshared: every sequence owns its own copy of the prefix blocks
    nbs = [-(-int(t) // B) for t in lens]
    tabs_u, off = [], 0
    for nb in nbs:
        tabs_u.append(list(range(off, off + nb)))
        off += nb
    kpu, vpu = place_contiguous(sk, sv, tabs_u, off, Hkv, D)
    # shared: the three prefix blocks are one physical copy
    npre = pre // B
    tabs_s, off = [], npre
    for nb in nbs:
        tabs_s.append(list(range(npre)) + list(range(off, off + nb - npre)))
        off += nb - npre
    kps, vps = place_contiguous(sk, sv, tabs_s, off, Hkv, D)
    def pack(tabs):
        t = np.full((len(tabs), max(nbs)), -1, np.int32)
        for i, r in enumerate(tabs):
            t[i, :len(r)] = r
        return t
    a = oracle.decode_attention(q, kpu, vpu, pack(tabs_u), lens, 0.4, "f32")
    b = oracle.decode_attention(q, kps, vps, pack(tabs_s), lens, 0.4, "f32")
    assert np.array_equal(a, b)


def test_split_and_merge_equals_unsplit():
    """[2] ("The Custom CUDA Kernel"): per-piece partial outputs and
    denominators merged stably reproduce the full softmax."""
    rng = np.random.default_rng(23)
    lens = [1, 16, 100, 513, 1030]
    q, kp, vp, tab, cl, sk, sv = random_paged_case(rng, lens, 4, 2, 16)
    full = oracle.decode_attention(q, kp, vp, tab, cl, 0.25, "f32")
    cut_rng = np.random.default_rng(24)
    def cuts(s, ctx):
        k = int(cut_rng.integers(0, 6))
        return sorted(set(int(c) for c in cut_rng.integers(1, max(ctx, 2), size=k) if 0 < c < ctx))
    split = oracle.decode_attention_split(q, kp, vp, tab, cl, 0.25, "f32", cuts)
    np.testing.assert_allclose(split, full, rtol=0, atol=1e-12)
    fixed = oracle.decode_attention_split(q, kp, vp, tab, cl, 0.25, "f32",
                                          lambda s, c: list(range(512, c, 512)))
    np.testing.assert_allclose(fixed, full, rtol=0, atol=1e-12)


def test_unused_slots_do_not_leak():
    rng = np.random.default_rng(25)
    q, kp, vp, tab, cl, sk, sv = random_paged_case(rng, [5, 17, 40], 2, 2, 8)
    a = oracle.decode_attention(q, kp, vp, tab, cl, 0.3, "f32")
    kp2 = np.where(np.isnan(kp), 1e30, kp)
    vp2 = np.where(np.isnan(vp), -1e30, vp)
    b = oracle.decode_attention(q, kp2, vp2, tab, cl, 0.3, "f32")
    assert np.isfinite(a).all() and np.array_equal(a, b)


# ---------------------------------------------------------------------------
# planted mistakes must be caught by the pins above
# ---------------------------------------------------------------------------
def _brute_pin_passes():
    rng = np.random.default_rng(31)
    lens = [5, 17, 40]
    D = 8
    q, kp, vp, tab, cl, sk, sv = random_paged_case(rng, lens, 4, 2, D)
    try:
        got = oracle.decode_attention(q, kp, vp, tab, cl, 1 / math.sqrt(D), "f32")
    except Exception:
        return False
    ref = brute_force(q, sk, sv, 1 / math.sqrt(D))
    return bool(np.all(np.abs(got - ref) <= 1e-12))


def test_pins_catch_planted_mistakes(monkeypatch):
    assert _brute_pin_passes()
    mistakes = {
        "head map hq % Hkv": ("_kv_head", lambda hq, Hq, Hkv: hq % Hkv),
        "block and offset swapped": ("slot_of", lambda row, p, b=16: int(row[p % b]) * b + p // b
                                     if p % b < len(row) else 0),
        "no masking of the last block": ("gather_sequence",
                                         lambda pool, row, ctx, b=16: np.concatenate(
                                             [pool[int(row[i])].transpose(1, 0, 2)
                                              for i in range(-(-ctx // b))])),
    }
    orig = {name: getattr(oa, name) for name, _ in mistakes.values()}
    for label, (name, fn) in mistakes.items():
        monkeypatch.setattr(oa, name, fn)
        assert not _brute_pin_passes(), f"planted mistake not caught: {label}"
        monkeypatch.setattr(oa, name, orig[name])
    assert _brute_pin_passes()


def test_planted_scale_and_transpose_mistakes_are_caught():
    rng = np.random.default_rng(32)
    q, kp, vp, tab, cl, sk, sv = random_paged_case(rng, [23], 2, 2, 8)
    ref = brute_force(q, sk, sv, 0.35)
    good = oracle.decode_attention(q, kp, vp, tab, cl, 0.35, "f32")
    assert np.abs(good - ref).max() <= 1e-12
    no_scale = oracle.decode_attention(q, kp, vp, tab, cl, 1.0, "f32")
    assert np.abs(no_scale - ref).max() > 1e-6
    swapped = oracle.decode_attention(q, vp, kp, tab, cl, 0.35, "f32")  # K and V exchanged
    assert np.abs(swapped - ref).max() > 1e-6


def test_swap_blocks_layout_and_round_trip():
    # host layout [n][layer][K, V][block bytes]: element (i, l, kv, h, r, d)
    # of the host copy is element (h, r, d) of block ids[i] in that pool
    rng = np.random.default_rng(3)
    L, NB, Hkv, B, D = 2, 6, 2, 4, 8
    kp = [rng.integers(0, 2 ** 16, size=(NB, Hkv, B, D)).astype(np.uint16) for _ in range(L)]
    vp = [rng.integers(0, 2 ** 16, size=(NB, Hkv, B, D)).astype(np.uint16) for _ in range(L)]
    ids = [4, 1, 9, 2]                       # 9 lies outside the pool
    host = oa.swap_out_blocks(kp, vp, ids)
    view = host.view(np.uint16).reshape(len(ids), L, 2, Hkv, B, D)
    for i, b in enumerate(ids):
        for l in range(L):
            for h in range(Hkv):
                for r in range(B):
                    for d in range(D):
                        if b >= NB:
                            assert view[i, l, 0, h, r, d] == 0 and view[i, l, 1, h, r, d] == 0
                        else:
                            assert view[i, l, 0, h, r, d] == kp[l][b, h, r, d]
                            assert view[i, l, 1, h, r, d] == vp[l][b, h, r, d]
    # swapping out of blocks a and back into blocks b is a block copy a -> b
    k2 = [x.copy() for x in kp]
    v2 = [x.copy() for x in vp]
    oa.swap_in_blocks(k2, v2, [0, 5, 3, 3], host)
    k3 = [x.copy() for x in kp]
    v3 = [x.copy() for x in vp]
    oa.copy_blocks(k3 + v3, [(4, 0), (1, 5), (2, 3)])
    # entry 2 (block 9) is skipped on the way out, so block 3 receives entry 3
    for a, b in zip(k2 + v2, k3 + v3):
        assert np.array_equal(a, b)
    # round trip into the same blocks changes nothing
    k4 = [x.copy() for x in kp]
    v4 = [x.copy() for x in vp]
    oa.swap_in_blocks(k4, v4, [4, 1, 2], host[[0, 1, 3]])
    for a, b in zip(k4 + v4, kp + vp):
        assert np.array_equal(a, b)
