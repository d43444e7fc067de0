"""Pins for the fp8 (E4M3) cache oracle (CPU only).

The code's values are pinned to the OCP E4M3 definition's fixed points and to
torch's float8_e4m3fn (an independent library implementation of the same
format); rounding to torch's conversion and to a brute-force nearest search;
saturation and NaN to closed forms; attention over an fp8 cache to a plain
loop over the dequantised, unpaged values.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oa
from oracle import fp8
from test_oracle_attention import brute_force, place_contiguous

B = 16


def test_fixed_points_of_the_format():
    v = fp8.e4m3_decode(np.arange(256))
    assert v[0x00] == 0.0 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x08] == 2.0 ** -6                       # smallest normal
    assert v[0x38] == 1.0 and v[0x3F] == 1.875 and v[0x40] == 2.0
    assert v[0x7E] == 448.0 and math.isnan(v[0x7F])
    assert v[0x80] == 0.0 and math.copysign(1.0, v[0x80]) == -1.0
    assert v[0xFE] == -448.0 and math.isnan(v[0xFF])
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                    # strictly increasing codes 0..0x7E
    assert np.array_equal(v[0x80:0xFF], -pos)


def test_decode_matches_torch_for_every_code():
    c = np.arange(256, dtype=np.uint8)
    t = torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
    v = fp8.e4m3_decode(c)
    assert np.array_equal(np.isnan(v), np.isnan(t))
    ok = ~np.isnan(v)
    assert np.array_equal(v[ok], t[ok])
    assert np.array_equal(np.signbit(v[ok]), np.signbit(t[ok]))


def _in_range_samples():
    rng = np.random.default_rng(5)
    pos = fp8.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2                    # exact ties
    near = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1000))])
    x = np.concatenate([pos, mids, near, rng.standard_normal(100_000) * 40,
                        rng.standard_normal(50_000) * 0.005, rng.uniform(-448, 448, 50_000)])
    x = x.astype(np.float32)
    x = x[np.abs(x) <= 448]
    return np.concatenate([x, -x])


def test_encode_matches_torch_in_range_including_ties():
    x = _in_range_samples()
    mine = fp8.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def test_encode_is_the_nearest_value_ties_to_even():
    x = _in_range_samples()[::7]
    vals = fp8.e4m3_decode(np.arange(0x7F))
    got = fp8.e4m3_decode(fp8.e4m3_encode(x))
    a = np.abs(x.astype(np.float64))
    d = np.abs(vals[None, :] - a[:, None])
    best = d.min(axis=1)
    assert np.array_equal(np.abs(np.abs(got) - a), best)
    # on a tie the chosen code is even
    ties = (d == best[:, None]).sum(axis=1) == 2
    assert ties.any()
    assert np.all(fp8.e4m3_encode(x[ties]) % 2 == 0)


def test_saturation_nan_and_signed_zero():
    x = np.array([448, 448.5, 464, 465, 1e6, np.inf], dtype=np.float32)
    assert np.all(fp8.e4m3_encode(x) == 0x7E)
    assert np.all(fp8.e4m3_encode(-x) == 0xFE)
    assert fp8.e4m3_encode(np.float32(np.nan)) == 0x7F
    assert fp8.e4m3_encode(-np.float32(np.nan)) == 0x7F
    assert fp8.e4m3_encode(np.float32(0.0)) == 0x00
    assert fp8.e4m3_encode(np.float32(-0.0)) == 0x80
    assert fp8.e4m3_encode(np.float32(-2.0 ** -11)) == 0x80   # rounds to -0
    assert fp8.e4m3_encode(np.float32(2.0 ** -10)) == 0x00    # tie 0 / 2^-9: even
    assert fp8.e4m3_encode(np.float32(3 * 2.0 ** -10)) == 0x02  # tie 1 / 2: even


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_quantize_with_a_scale_matches_torch(dtype):
    rng = np.random.default_rng(7)
    x32 = (rng.standard_normal(20_000) * 3).astype(np.float32)
    if dtype == "bf16":
        stored = (torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy()
                  .view(np.uint16))
        xt = torch.from_numpy(stored.view(np.int16)).view(torch.bfloat16).float()
    elif dtype == "f16":
        stored = x32.astype(np.float16)
        xt = torch.from_numpy(stored).float()
    else:
        stored = x32
        xt = torch.from_numpy(stored)
    for scale in (1.0, 0.0123, 1 / 64, 3.7):
        ref = (xt / torch.tensor(scale, dtype=torch.float32)).to(torch.float8_e4m3fn)
        got = fp8.quantize(stored, dtype, scale)
        r = ref.view(torch.uint8).numpy()
        inside = np.abs((xt / np.float32(scale)).numpy()) <= 448
        assert np.array_equal(got[inside], r[inside])
        assert np.all(got[~inside] % 128 == 0x7E)


def test_round_trip_error_bound():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(50_000) * 2).astype(np.float32)
    scale = 4.0 / 448
    back = fp8.dequantize(fp8.quantize(x, "f32", scale), scale)
    y = np.abs(x.astype(np.float64)) / np.float32(scale)
    err = np.abs(back - x)
    normal = (y >= 2.0 ** -6) & (y <= 448)
    sub = y < 2.0 ** -6
    # half an ulp: 2^-4 relative for normals, 2^-10 absolute (times scale) below
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x[normal]) * (1 + 1e-6))
    assert np.all(err[sub] <= 2.0 ** -10 * scale * (1 + 1e-6))
    # beyond the range the value saturates at 448 * scale
    assert np.all(np.abs(back[y > 448]) == 448 * float(np.float32(scale)))
    assert normal.sum() > 40_000 and (y > 448).any()


def test_cache_write_places_quantised_rows():
    rng = np.random.default_rng(9)
    NB, Hkv, D = 4, 2, 8
    kp = np.zeros((NB, Hkv, B, D), np.uint8)
    vp = np.zeros((NB, Hkv, B, D), np.uint8)
    kn = rng.standard_normal((3, Hkv, D)).astype(np.float32)
    vn = rng.standard_normal((3, Hkv, D)).astype(np.float32)
    fp8.reshape_and_cache_fp8(kn, vn, kp, vp, [3 * B + 5, -1, 0 * B + 15], "f32", 0.5, 0.25)
    assert np.array_equal(kp[3, :, 5, :], fp8.quantize(kn[0], "f32", 0.5))
    assert np.array_equal(vp[0, :, 15, :], fp8.quantize(vn[2], "f32", 0.25))
    written = np.zeros((NB, B), bool)
    written[3, 5] = written[0, 15] = True
    assert not kp.transpose(0, 2, 1, 3)[~written].any()
    assert not vp.transpose(0, 2, 1, 3)[~written].any()


def test_attention_over_an_fp8_cache_is_the_plain_definition():
    rng = np.random.default_rng(12)
    lens = [5, 16, 17, 40]
    Hq, Hkv, D = 4, 2, 8
    ks, vs = 0.03, 0.011
    seqs_k = [rng.integers(0, 256, (t, Hkv, D)).astype(np.uint8) for t in lens]
    seqs_v = [rng.integers(0, 256, (t, Hkv, D)).astype(np.uint8) for t in lens]
    for a in seqs_k + seqs_v:          # no NaN codes in live rows
        a[(a & 0x7F) == 0x7F] = 0x3F
    nbs = [-(-t // B) for t in lens]
    NB = sum(nbs) + 2
    perm = rng.permutation(NB)
    tab = np.full((len(lens), max(nbs)), -1, np.int32)
    tables, off = [], 0
    for s, nb in enumerate(nbs):
        tab[s, :nb] = perm[off:off + nb]
        tables.append(list(perm[off:off + nb]))
        off += nb
    kp, vp = place_contiguous(seqs_k, seqs_v, tables, NB, Hkv, D, fill=0x7F, dtype=np.uint8)
    q = rng.standard_normal((len(lens), Hq, D)).astype(np.float32)
    got = oracle.decode_attention(q, kp, vp, tab, np.array(lens, np.int32), 0.3, "f32",
                                  kv_dtype="e4m3", k_scale=ks, v_scale=vs)
    sk = [fp8.e4m3_decode(k) * float(np.float32(ks)) for k in seqs_k]
    sv = [fp8.e4m3_decode(v) * float(np.float32(vs)) for v in seqs_v]
    ref = brute_force(q.astype(np.float64), sk, sv, 0.3)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    # a planted mistake - the V scale applied to K - is caught
    bad = oracle.decode_attention(q, kp, vp, tab, np.array(lens, np.int32), 0.3, "f32",
                                  kv_dtype="e4m3", k_scale=vs, v_scale=vs)
    assert np.abs(bad - ref).max() > 1e-6


def test_widen_e4m3():
    assert oa.widen(np.array([0x38, 0xC0], np.uint8), "e4m3").tolist() == [1.0, -2.0]
