"""Pins for the chunked-prefill attention oracle (CPU only).

A chunk of one token per sequence is the decode oracle; a plain loop over
unpaged arrays with the causal rule written out, and torch's fp64 SDPA with an
explicit mask, give the same values; cutting a chunk in two changes nothing.
"""
import numpy as np
import pytest
import torch

import oracle
from test_oracle_attention import place_contiguous

B = 16


def paged_prefill_case(rng, prev, chunk, Hq, Hkv, D, extra_blocks=3):
    """Random unpaged K/V per sequence (length prev + chunk), placed in a
    shuffled pool; packed queries for the chunks."""
    lens = [p + c for p, c in zip(prev, chunk)]
    seqs_k = [rng.standard_normal((t, Hkv, D)) for t in lens]
    seqs_v = [rng.standard_normal((t, Hkv, D)) for t in lens]
    nbs = [-(-t // B) for t in lens]
    NB = sum(nbs) + extra_blocks
    perm = rng.permutation(NB)
    tab = np.full((len(lens), max(nbs + [1])), -1, np.int32)
    tables, off = [], 0
    for s, nb in enumerate(nbs):
        tab[s, :nb] = perm[off:off + nb]
        tables.append(list(perm[off:off + nb]))
        off += nb
    kp, vp = place_contiguous(seqs_k, seqs_v, tables, NB, Hkv, D)
    q_start = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    q = rng.standard_normal((int(q_start[-1]), Hq, D))
    return q, q_start, kp, vp, tab, np.array(lens, np.int32), seqs_k, seqs_v


def causal_brute_force(q, q_start, seqs_k, seqs_v, scale, Hq, shift=0):
    """Plain loops: row i of sequence s's chunk attends to keys 0..prev+i
    (0..prev+i+shift for a planted mistake; rows left with no key stay 0)."""
    T, _, D = q.shape
    out = np.zeros((T, Hq, D))
    for s in range(len(q_start) - 1):
        K, V = seqs_k[s], seqs_v[s]
        L = len(K)
        C = int(q_start[s + 1] - q_start[s])
        Hkv = K.shape[1]
        for i in range(C):
            r = int(q_start[s]) + i
            last = min(L - C + i + shift, L - 1)
            if last < 0:
                continue
            for hq in range(Hq):
                h = hq // (Hq // Hkv)
                z = [scale * sum(float(q[r, hq, d]) * float(K[j, h, d]) for d in range(D))
                     for j in range(last + 1)]
                m = max(z)
                w = [np.exp(v - m) for v in z]
                tot = sum(w)
                for d in range(D):
                    out[r, hq, d] = sum(w[j] * float(V[j, h, d]) for j in range(last + 1)) / tot
    return out


def test_chunk_of_one_token_is_the_decode_oracle():
    rng = np.random.default_rng(60)
    prev = [4, 0, 16, 39, 100]
    q, qs, kp, vp, tab, lens, _, _ = paged_prefill_case(rng, prev, [1] * 5, 8, 2, 16)
    a = oracle.prefill_attention(q, qs, kp, vp, tab, lens, 0.2, "f32")
    b = oracle.decode_attention(q, kp, vp, tab, lens, 0.2, "f32")
    assert np.array_equal(a, b)


def test_matches_a_plain_causal_loop():
    rng = np.random.default_rng(61)
    prev, chunk = [0, 5, 17, 30], [7, 1, 16, 3]
    Hq, Hkv, D = 4, 2, 8
    q, qs, kp, vp, tab, lens, sk, sv = paged_prefill_case(rng, prev, chunk, Hq, Hkv, D)
    got = oracle.prefill_attention(q.astype(np.float32), qs, kp.astype(np.float32),
                                   vp.astype(np.float32), tab, lens, 0.3, "f32")
    q32 = q.astype(np.float32).astype(np.float64)
    sk32 = [k.astype(np.float32).astype(np.float64) for k in sk]
    sv32 = [v.astype(np.float32).astype(np.float64) for v in sv]
    ref = causal_brute_force(q32, qs, sk32, sv32, 0.3, Hq)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    # planted off-by-ones (the query's own key left out, the next key let in) are caught
    for shift in (-1, 1):
        bad = causal_brute_force(q32, qs, sk32, sv32, 0.3, Hq, shift=shift)
        assert np.abs(bad - got).max() > 1e-3


def test_matches_torch_sdpa_with_an_explicit_mask():
    rng = np.random.default_rng(62)
    prev, chunk = [10, 64, 0], [20, 33, 48]
    Hq, Hkv, D = 8, 2, 32
    q, qs, kp, vp, tab, lens, sk, sv = paged_prefill_case(rng, prev, chunk, Hq, Hkv, D)
    got = oracle.prefill_attention(q, qs, kp, vp, tab, lens, 0.11, "f32")
    for s in range(len(prev)):
        L, C = int(lens[s]), chunk[s]
        K = torch.from_numpy(np.repeat(sk[s], Hq // Hkv, axis=1)).permute(1, 0, 2)   # [Hq, L, D]
        V = torch.from_numpy(np.repeat(sv[s], Hq // Hkv, axis=1)).permute(1, 0, 2)
        Q = torch.from_numpy(q[qs[s]:qs[s + 1]]).permute(1, 0, 2)                  # [Hq, C, D]
        mask = torch.from_numpy(np.arange(L)[None, :] <= (L - C + np.arange(C))[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask,
                                                               scale=0.11)
        np.testing.assert_allclose(got[qs[s]:qs[s + 1]], ref.permute(1, 0, 2).numpy(),
                                   rtol=0, atol=1e-12)


@pytest.mark.parametrize("cut", [1, 5, 16])
def test_two_chunks_equal_one(cut):
    rng = np.random.default_rng(63 + cut)
    prev, chunk = [7], [24]
    q, qs, kp, vp, tab, lens, _, _ = paged_prefill_case(rng, prev, chunk, 4, 1, 8)
    whole = oracle.prefill_attention(q, qs, kp, vp, tab, lens, 0.25, "f32")
    first = oracle.prefill_attention(q[:cut], np.array([0, cut], np.int32), kp, vp, tab,
                                     np.array([prev[0] + cut], np.int32), 0.25, "f32")
    second = oracle.prefill_attention(q[cut:], np.array([0, 24 - cut], np.int32), kp, vp, tab,
                                      lens, 0.25, "f32")
    np.testing.assert_allclose(np.concatenate([first, second]), whole, rtol=0, atol=1e-14)


def test_rows_subset_and_empty_chunks():
    rng = np.random.default_rng(64)
    q, qs, kp, vp, tab, lens, _, _ = paged_prefill_case(rng, [3, 9, 2], [4, 0, 2], 2, 1, 4)
    full = oracle.prefill_attention(q, qs, kp, vp, tab, lens, 0.5, "f32")
    part = oracle.prefill_attention(q, qs, kp, vp, tab, lens, 0.5, "f32", rows=[1, 5])
    assert np.array_equal(part[[1, 5]], full[[1, 5]])
    assert np.isnan(part[[0, 2, 3, 4]]).all()
    with pytest.raises(ValueError):
        oracle.prefill_attention(q, qs, kp, vp, tab, np.array([3, 9, 1], np.int32), 0.5, "f32")


def test_fp8_cache_is_the_16bit_oracle_on_dequantised_values():
    from oracle import fp8
    from oracle import attention as oa
    rng = np.random.default_rng(65)
    prev, chunk = [9, 0, 30], [5, 12, 3]
    Hq, Hkv, D = 4, 2, 8
    _, qs, kp, vp, tab, lens, _, _ = paged_prefill_case(rng, prev, chunk, Hq, Hkv, D)
    codes_k = rng.integers(0, 256, kp.shape).astype(np.uint8)
    codes_v = rng.integers(0, 256, vp.shape).astype(np.uint8)
    for c in (codes_k, codes_v):
        c[(c & 0x7F) == 0x7F] = 0x30            # no NaN codes
    q = rng.standard_normal((int(qs[-1]), Hq, D)).astype(np.float32)
    got = oracle.prefill_attention(q, qs, codes_k, codes_v, tab, lens, 0.4, "f32",
                                   kv_dtype="e4m3", k_scale=0.125, v_scale=3.0)
    ref = oracle.prefill_attention(q, qs, fp8.dequantize(codes_k, 0.125),
                                   fp8.dequantize(codes_v, 3.0), tab, lens, 0.4, "f32")
    np.testing.assert_allclose(got, ref, rtol=0, atol=0)
    # the decode oracle agrees on one-row chunks of the same cache
    ones = np.arange(4, dtype=np.int32)
    d = oracle.decode_attention(q[:3], codes_k, codes_v, tab, lens, 0.4, "f32",
                                kv_dtype="e4m3", k_scale=0.125, v_scale=3.0)
    p1 = oracle.prefill_attention(q[:3], ones, codes_k, codes_v, tab, lens, 0.4, "f32",
                                  kv_dtype="e4m3", k_scale=0.125, v_scale=3.0)
    assert np.array_equal(d, p1)
    assert oa.widen(codes_k[0, 0, 0, :2], "e4m3").shape == (2,)
