"""GPU parity of the shared-prefix decode step over an fp8 (E4M3) cache
(kv_paged_attention_decode_append_shared_fp8) against the oracle: the shared
positions read once for the batch ("PagedAttention - how vLLM stopped wasting
80% of your GPU memory", "Memory sharing") from pools of E4M3 codes with one
scale per pool ("How does this relate to quantization?"). Slots and both pools
(the new token quantised into its slot) bit exact against the oracle's write;
the output within the 16-bit tolerance of the oracle's float64 attention over
the dequantised cache.
"""
import numpy as np
import pytest

import oracle
from oracle import attention as oa
from oracle import fp8 as ofp8
from workloads import round_to_dtype
from gpu_common import check_attention, log, to_dev, to_host, bits, POISON

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_162_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


def kvlib():
    import paged_kv_cache_162_amd as kv
    return kv


FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)


def shared_case_fp8(rng, S, shared_blocks, tails, Hq, Hkv, D, dt, B=16):
    """S sequences sharing their first shared_blocks blocks, then private tails; pools of
    random finite E4M3 codes (zeros and subnormals included), shuffled, every unused slot
    holding the NaN code."""
    lens = [shared_blocks * B + t for t in tails]
    tail_nbs = [-(-t // B) if t > 0 else 0 for t in tails]
    NB = shared_blocks + sum(tail_nbs) + 7
    perm = rng.permutation(NB)
    tab = np.full((S, shared_blocks + max(tail_nbs + [1])), -1, np.int32)
    off = shared_blocks
    for s in range(S):
        tab[s, :shared_blocks] = perm[:shared_blocks]
        tab[s, shared_blocks:shared_blocks + tail_nbs[s]] = perm[off:off + tail_nbs[s]]
        off += tail_nbs[s]
    kp = rng.choice(FINITE, (NB, Hkv, B, D))
    vp = rng.choice(FINITE, (NB, Hkv, B, D))
    live = np.zeros((NB, B), bool)
    for s, t in enumerate(lens):
        for p_ in range(t):
            live[tab[s, p_ // B], p_ % B] = True
    dead = np.argwhere(~live)
    for pool in (kp, vp):
        pool[dead[:, 0], :, dead[:, 1], :] = POISON["e4m3"]
    q = round_to_dtype(rng.standard_normal((S, Hq, D)).astype(np.float32), dt)
    return q, kp, vp, tab, np.array(lens, np.int32)


def run_shared_fp8(rng, dt, G, B, P, plan, S, Hkv, shared_blocks, tails, ks=0.07, vs=0.013,
                   cl_run=None, D=128):
    """One fused fp8 shared-prefix step; returns (out, slots, k pool, v pool) from the device
    and the inputs. cl_run optionally replaces the context lengths passed to the call."""
    kv = kvlib()
    q, kp, vp, tab, cl = shared_case_fp8(rng, S, shared_blocks, tails, G * Hkv, Hkv, D, dt, B)
    cl = cl if cl_run is None else cl_run
    shared = shared_blocks * B
    scale = float(np.float32(1 / np.sqrt(D)))
    kn = round_to_dtype(rng.standard_normal((S, Hkv, D)).astype(np.float32) * 2, dt)
    vn = round_to_dtype(rng.standard_normal((S, Hkv, D)).astype(np.float32) * 2, dt)
    tail_lens = np.maximum(cl - shared, 0)
    mt = int(tail_lens.max())
    wsb = kv.kv_paged_attention_workspace_bytes(S, G * Hkv, Hkv, D, mt, P)
    ws = torch.full((max(wsb, 16) // 4,), float("nan"), dtype=torch.float32,
                    device="cuda") if wsb else None
    aux = torch.full((kv.kv_paged_attention_shared_aux_bytes(S, G * Hkv, Hkv, D, shared) // 4,),
                     float("nan"), dtype=torch.float32, device="cuda")
    items = torch.from_numpy(kv.kv_paged_attention_plan(tail_lens, P)).cuda() if plan else None
    dk, dv = to_dev(kp, "e4m3"), to_dev(vp, "e4m3")
    out = torch.full((S, G * Hkv, D), float("nan"), dtype=torch.float32, device="cuda")
    slots = torch.full((S,), 7, dtype=torch.int64, device="cuda")
    log(f"[gpu] shared prefix fp8 {dt} S={S} G={G} Hkv={Hkv} B={B} shared={shared} P={P} "
        f"plan={plan}")
    kv.kv_paged_attention_decode_append_shared_fp8(
        out, to_dev(q, dt), to_dev(kn, dt), to_dev(vn, dt), dk, dv,
        torch.from_numpy(tab).cuda(), torch.from_numpy(cl).cuda(), scale, ks, vs, shared, mt,
        slots, aux, ws, P, items)
    torch.cuda.synchronize()
    dev = (out.cpu().numpy(), slots.cpu().numpy(), to_host(dk, "e4m3"), to_host(dv, "e4m3"))
    return dev, (q, kp, vp, tab, cl, kn, vn, scale)


# (query dtype, group, block size, partition, plan): every group size runs the MFMA tail
# kernel over fp8; a partition below the 700-token tail makes the merge kernel combine
CASES = [("bf16", 8, 16, 0, True), ("bf16", 8, 16, 256, False), ("f16", 4, 16, 128, True),
         ("bf16", 16, 16, 0, True), ("bf16", 8, 8, 0, True), ("bf16", 4, 32, 64, True),
         ("bf16", 1, 16, 0, True), ("f16", 1, 8, 128, False), ("f16", 2, 16, 0, False),
         ("bf16", 6, 16, 0, True), ("f16", 3, 32, 128, False)]


@pytest.mark.parametrize("dt,G,B,P,plan", CASES)
def test_shared_prefix_fp8_step_against_oracle(dt, G, B, P, plan):
    rng = np.random.default_rng(9500 + CASES.index((dt, G, B, P, plan)))
    S, Hkv = 37, 2
    # 664 / 656 / 640 shared positions: two ranges, the second ragged
    shared_blocks = {8: 83, 16: 41, 32: 20}[B]
    tails = list(rng.integers(1, 300, S))
    tails[0], tails[1], tails[2] = 1, 2, 700       # new token only; tiny; several partitions
    ks, vs = 0.07, 0.013
    (out, slots, dk, dv), (q, kp, vp, tab, cl, kn, vn, scale) = run_shared_fp8(
        rng, dt, G, B, P, plan, S, Hkv, shared_blocks, tails, ks, vs)
    ref_slots = oa.slot_mapping(tab, np.arange(S), cl - 1, block_size=B)
    rk, rv = kp.copy(), vp.copy()
    ofp8.reshape_and_cache_fp8(kn, vn, rk, rv, ref_slots, dt, ks, vs, block_size=B)
    ref = oracle.decode_attention(q, rk, rv, tab, cl, scale, dt, block_size=B, kv_dtype="e4m3",
                                  k_scale=ks, v_scale=vs)
    assert np.array_equal(slots, ref_slots)
    assert np.array_equal(dk, rk) and np.array_equal(dv, rv)
    log(check_attention(out.reshape(-1, 128), ref.reshape(-1, 128), dt,
                        f"shared fp8 {dt} G={G} B={B} P={P} plan={plan}"))


# Shapes of the prefix pass's plan (sequences, group, KV heads, block size, shared blocks):
# 16 column tiles per head; 8,192 positions in 4 ranges of slices of 256; the longest shared
# prefix, 131,072 positions in 16 ranges of 8 slices of 1,024; 104 positions of 8-token blocks
PLANS = [(64, 4, 8, 16, 128), (32, 4, 8, 16, 512), (2, 1, 1, 32, 4096), (3, 16, 1, 8, 13)]


@pytest.mark.parametrize("S,G,Hkv,B,shared_blocks", PLANS)
def test_shared_prefix_fp8_plans(S, G, Hkv, B, shared_blocks):
    rng = np.random.default_rng(9600 + S + G + shared_blocks)
    tails = list(rng.integers(1, 90, S))
    tails[0] = 1
    ks, vs = 0.25, 0.25
    (out, slots, dk, dv), (q, kp, vp, tab, cl, kn, vn, scale) = run_shared_fp8(
        rng, "bf16", G, B, 0, True, S, Hkv, shared_blocks, tails, ks, vs)
    ref_slots = oa.slot_mapping(tab, np.arange(S), cl - 1, block_size=B)
    rk, rv = kp.copy(), vp.copy()
    ofp8.reshape_and_cache_fp8(kn, vn, rk, rv, ref_slots, "bf16", ks, vs, block_size=B)
    ref = oracle.decode_attention(q, rk, rv, tab, cl, scale, "bf16", block_size=B,
                                  kv_dtype="e4m3", k_scale=ks, v_scale=vs)
    assert np.array_equal(slots, ref_slots)
    assert np.array_equal(dk, rk) and np.array_equal(dv, rv)
    check_attention(out.reshape(-1, 128), ref.reshape(-1, 128), "bf16",
                    f"shared fp8 plan S={S} G={G} Hkv={Hkv} B={B} shared={shared_blocks * B}")


def test_shared_prefix_fp8_edge_lengths():
    """A sequence of exactly the shared length gets the attention over the shared positions
    and no write; a shorter one gets NaN; the others are unaffected."""
    rng = np.random.default_rng(9700)
    dt, Hkv, G, B, S, shared_blocks = "bf16", 2, 8, 16, 5, 8
    tails = [5, 9, 1, 30, 17]
    shared = shared_blocks * B
    cl_run = np.array([shared + t for t in tails], np.int32)
    cl_run[1] = shared          # prefix only
    cl_run[3] = shared - 3      # shorter than the shared part: invalid
    ks, vs = 0.05, 0.02
    (out, slots, dk, dv), (q, kp, vp, tab, cl, kn, vn, scale) = run_shared_fp8(
        rng, dt, G, B, 0, False, S, Hkv, shared_blocks, tails, ks, vs, cl_run=cl_run)
    ok = [0, 2, 4]
    ref_slots = oa.slot_mapping(tab[ok], np.arange(len(ok)), cl[ok] - 1, block_size=B)
    rk, rv = kp.copy(), vp.copy()
    ofp8.reshape_and_cache_fp8(kn[ok], vn[ok], rk, rv, ref_slots, dt, ks, vs, block_size=B)
    ref = oracle.decode_attention(q[ok], rk, rv, tab[ok], cl[ok], scale, dt, block_size=B,
                                  kv_dtype="e4m3", k_scale=ks, v_scale=vs)
    ref1 = oracle.decode_attention(q[[1]], kp, vp, tab[[1]], cl[[1]], scale, dt, block_size=B,
                                   kv_dtype="e4m3", k_scale=ks, v_scale=vs)
    assert np.array_equal(slots[ok], ref_slots) and slots[1] == -1 and slots[3] == -1
    assert np.isnan(out[3]).all()
    check_attention(out[ok].reshape(-1, 128), ref.reshape(-1, 128), dt, "valid rows")
    check_attention(out[1].reshape(-1, 128), ref1.reshape(-1, 128), dt, "prefix only")
    assert np.array_equal(dk, rk) and np.array_equal(dv, rv)


@pytest.mark.parametrize("B", [16, 32])
def test_session_shared_fp8_step_matches_plain_step(B):
    """Workload prefix-share-long-fp8 (64 sequences sharing 4,096 positions of an fp8
    cache) through the session: it takes the shared-prefix step by itself; against its plain
    fused step, identical slots and pools, outputs within the tolerance of each other and of
    the oracle (every output)."""
    from gpu_common import Case
    res = {}
    for shared in (True, False):
        case = Case(11, block_size=B)
        log(f"[gpu] session workload 11 B={B} shared_prefix={shared}")
        case.device_run(shared_prefix=shared)
        assert (case.sess.shared_tokens == 4096) == shared
        res[shared] = (case.out_dev.cpu().numpy(), to_host(case.k_dev, "e4m3"),
                       to_host(case.v_dev, "e4m3"), case.sess.d_slots.cpu().numpy())
        case.sess.close()
    a, b = res[True], res[False]
    assert np.array_equal(a[3], b[3]) and np.array_equal(a[3], case.step_slots)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
    assert np.array_equal(a[1], case.k_ref) and np.array_equal(a[2], case.v_ref)
    D = case.sp.D
    check_attention(a[0].reshape(-1, D), b[0].reshape(-1, D), case.dt, "shared vs plain step")
    ref = case.oracle_out()
    log(check_attention(a[0].reshape(-1, D), ref.reshape(-1, D), case.dt,
                        "shared fp8 step vs oracle"))


def test_shared_fp8_step_graph_replay_matches_eager():
    """The fp8 shared-prefix step captured in a HIP graph (no memset nodes): every replay,
    with the outputs, slots and scratch poisoned in between by eager work, reproduces the
    eager step bit for bit (outputs, both pools, slots)."""
    from gpu_common import Case
    case = Case(11)
    case.device_run()
    sess = case.sess
    assert sess.shared_tokens == 4096
    eager = (case.out_dev.cpu().numpy().copy(), to_host(case.k_dev, "e4m3").copy(),
             to_host(case.v_dev, "e4m3").copy(), sess.d_slots.cpu().numpy().copy())
    out = torch.full_like(case.out_dev, float("nan"))
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            sess.step(case.q_dev, case.kn_dev, case.vn_dev, out, case.sp.scale)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        sess.d_slots.fill_(-7)
        sess.aux.fill_(float("nan"))
        if sess.workspace is not None:
            sess.workspace.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"[gpu] shared fp8 step graph replay {rep}")
        assert np.array_equal(out.cpu().numpy().view(np.uint32), eager[0].view(np.uint32))
        assert np.array_equal(to_host(case.k_dev, "e4m3"), eager[1])
        assert np.array_equal(to_host(case.v_dev, "e4m3"), eager[2])
        assert np.array_equal(sess.d_slots.cpu().numpy(), eager[3])
    sess.close()


@pytest.mark.parametrize("case", range(4))
def test_shared_prefix_fp8_random_shapes(case):
    """Seeded random shapes of the fp8 shared step: group size, block size, sequences, shared
    length, tail lengths, partition size, plan and scales; slots and pools bit exact, every
    output within tolerance."""
    rng = np.random.default_rng(9800 + case)
    G = int(rng.choice([1, 2, 4, 5, 8, 16]))
    B = int(rng.choice([8, 16, 32]))
    dt = str(rng.choice(["bf16", "f16"]))
    S = int(rng.integers(2, 40))
    Hkv = int(rng.choice([1, 2, 4]))
    shared_blocks = int(rng.integers(1, 1600 // B))
    tails = [int(t) for t in rng.integers(1, 400, S)]
    P = int(rng.choice([0, 64, 128, 256]))
    plan = bool(rng.integers(0, 2))
    ks, vs = float(rng.uniform(0.01, 1.0)), float(rng.uniform(0.01, 1.0))
    (out, slots, dk, dv), (q, kp, vp, tab, cl, kn, vn, scale) = run_shared_fp8(
        rng, dt, G, B, P, plan, S, Hkv, shared_blocks, tails, ks, vs)
    ref_slots = oa.slot_mapping(tab, np.arange(S), cl - 1, block_size=B)
    rk, rv = kp.copy(), vp.copy()
    ofp8.reshape_and_cache_fp8(kn, vn, rk, rv, ref_slots, dt, ks, vs, block_size=B)
    ref = oracle.decode_attention(q, rk, rv, tab, cl, scale, dt, block_size=B, kv_dtype="e4m3",
                                  k_scale=ks, v_scale=vs)
    assert np.array_equal(slots, ref_slots)
    assert np.array_equal(dk, rk) and np.array_equal(dv, rv)
    check_attention(out.reshape(-1, 128), ref.reshape(-1, 128), dt,
                    f"shared fp8 random {case}: {dt} G={G} Hkv={Hkv} B={B} S={S} "
                    f"shared={shared_blocks * B} P={P} plan={plan}")


@pytest.mark.parametrize("where", ["prefix", "tail"])
def test_shared_fp8_step_invalid_table_entry(where):
    """Over an fp8 cache as over a 16-bit one: an out-of-pool block ID in the shared part of
    row 0's table makes every output NaN; one in a sequence's tail makes only that sequence
    NaN, the other outputs matching the oracle (no load leaves the pool)."""
    kv = kvlib()
    rng = np.random.default_rng(9900)
    dt, D, Hkv, G, B = "bf16", 128, 2, 8, 16
    S, shared_blocks = 6, 20
    tails = [40, 3, 77, 16, 1, 130]
    q, kp, vp, tab, cl = shared_case_fp8(rng, S, shared_blocks, tails, G * Hkv, Hkv, D, dt, B)
    shared = shared_blocks * B
    scale, ks, vs = 0.088, 0.06, 0.03
    kn = round_to_dtype(rng.standard_normal((S, Hkv, D)).astype(np.float32), dt)
    vn = round_to_dtype(rng.standard_normal((S, Hkv, D)).astype(np.float32), dt)
    bad_tab = tab.copy()
    victim = 2
    if where == "prefix":
        bad_tab[0, 7] = kp.shape[0] + 5          # only row 0's copy is read for the prefix
    else:
        bad_tab[victim, shared_blocks + 2] = -3  # a tail block of sequence 2
    ref_slots = oa.slot_mapping(tab, np.arange(S), cl - 1, block_size=B)
    rk, rv = kp.copy(), vp.copy()
    ofp8.reshape_and_cache_fp8(kn, vn, rk, rv, ref_slots, dt, ks, vs, block_size=B)
    ref = oracle.decode_attention(q, rk, rv, tab, cl, scale, dt, block_size=B, kv_dtype="e4m3",
                                  k_scale=ks, v_scale=vs)
    mt = int(max(cl - shared))
    wsb = kv.kv_paged_attention_workspace_bytes(S, G * Hkv, Hkv, D, mt, 0)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda") if wsb else None
    aux = torch.empty(kv.kv_paged_attention_shared_aux_bytes(S, G * Hkv, Hkv, D, shared) // 4,
                      dtype=torch.float32, device="cuda")
    out = torch.full((S, G * Hkv, D), 3.0, dtype=torch.float32, device="cuda")
    slots = torch.full((S,), 7, dtype=torch.int64, device="cuda")
    log(f"[gpu] shared fp8 step, invalid entry in the {where}")
    kv.kv_paged_attention_decode_append_shared_fp8(
        out, to_dev(q, dt), to_dev(kn, dt), to_dev(vn, dt), to_dev(kp, "e4m3"),
        to_dev(vp, "e4m3"), torch.from_numpy(bad_tab).cuda(), torch.from_numpy(cl).cuda(), scale,
        ks, vs, shared, mt, slots, aux, ws, 0, None)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    if where == "prefix":
        assert np.isnan(got).all()
    else:
        ok = [s for s in range(S) if s != victim]
        assert np.isnan(got[victim]).all()
        check_attention(got[ok].reshape(-1, D), ref[ok].reshape(-1, D), dt, "other sequences")
