"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact for slot mapping, the cache scatter and block copies; attention
within max |err| <= 1e-5 (fp32 inputs) or max |err| / RMS(oracle) <= 2e-3
(fp16/bf16 inputs). Every workload runs through the same session code the
benchmark times.
"""
import numpy as np
import pytest

import oracle
from oracle import attention as oa
from workloads import round_to_dtype
from gpu_common import (Case, check_attention, log, to_dev, to_host, bits, POISON)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_162_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


def kvlib():
    import paged_kv_cache_162_amd as kv
    return kv


# ---------------------------------------------------------------------------
# integer and byte work: bit exact
# ---------------------------------------------------------------------------
def test_slot_mapping_bit_exact():
    kv = kvlib()
    rng = np.random.default_rng(7)
    rows, maxb = 37, 9
    tables = rng.integers(-1, 5000, size=(rows, maxb)).astype(np.int32)
    n = 4099
    seq = rng.integers(-2, rows + 2, size=n).astype(np.int32)
    pos = rng.integers(-3, maxb * 16 + 5, size=n).astype(np.int32)
    log("[gpu] slot mapping n=%d" % n)
    d_slots = torch.empty(n, dtype=torch.int64, device="cuda")
    kv.kv_slot_mapping(torch.from_numpy(tables).cuda(), torch.from_numpy(seq).cuda(),
                       torch.from_numpy(pos).cuda(), d_slots)
    got = d_slots.cpu().numpy()
    ok = (seq >= 0) & (seq < rows)
    ref = np.full(n, -1, np.int64)
    ref[ok] = oa.slot_mapping(tables, seq[ok], pos[ok])
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("dt,D", [("f32", 64), ("f16", 128), ("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_reshape_and_cache_bit_exact(dt, D):
    kv = kvlib()
    rng = np.random.default_rng(11)
    NB, Hkv, n = 50, 3, 123
    store = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}[dt]
    nb = np.dtype(store).itemsize
    kp = rng.integers(0, 2 ** (8 * nb), size=(NB, Hkv, 16, D), dtype=np.uint64).astype(store)
    vp = rng.integers(0, 2 ** (8 * nb), size=(NB, Hkv, 16, D), dtype=np.uint64).astype(store)
    kn = rng.integers(0, 2 ** (8 * nb), size=(n, Hkv, D), dtype=np.uint64).astype(store)
    vn = rng.integers(0, 2 ** (8 * nb), size=(n, Hkv, D), dtype=np.uint64).astype(store)
    slots = rng.choice(NB * 16, size=n, replace=False).astype(np.int64)
    slots[::17] = -1
    slots[5] = NB * 16 + 3  # out of range: skipped
    view = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dt]
    log(f"[gpu] reshape_and_cache {dt} D={D} n={n}")
    dk, dv = to_dev(kp.view(view), dt), to_dev(vp.view(view), dt)
    kv.kv_reshape_and_cache(to_dev(kn.view(view), dt), to_dev(vn.view(view), dt), dk, dv,
                            torch.from_numpy(slots).cuda())
    ok = (slots >= 0) & (slots < NB * 16)
    rk, rv = kp.copy().view(view), vp.copy().view(view)
    oa.reshape_and_cache(kn.view(view)[ok], vn.view(view)[ok], rk, rv, slots[ok])
    assert np.array_equal(bits(to_host(dk, dt)), bits(rk))
    assert np.array_equal(bits(to_host(dv, dt)), bits(rv))


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("f32", 64), ("f16", 128)])
def test_append_tokens_bit_exact(dt, D):
    """Slot mapping + cache write in one launch: slots equal the oracle's slot
    formula, and the pools equal the oracle's scatter, bit for bit."""
    kv = kvlib()
    rng = np.random.default_rng(13)
    rows, maxb, NB, Hkv = 29, 7, 64, 4
    store = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}[dt]
    view = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dt]
    nb = np.dtype(store).itemsize
    # distinct physical blocks per table entry, with some holes (-1)
    tables = rng.permutation(NB * 8)[: rows * maxb].reshape(rows, maxb).astype(np.int32) % NB
    tables = np.where(rng.random((rows, maxb)) < 0.1, -1, tables).astype(np.int32)
    # one token per row at distinct (row, position) pairs so slots never repeat
    seq = np.arange(rows, dtype=np.int32)
    pos = rng.integers(0, maxb * 16, size=rows).astype(np.int32)
    pos[3], seq[4] = -1, rows + 5          # unmappable: slot -1, nothing written
    ref_slots = np.full(rows, -1, np.int64)
    okr = (seq >= 0) & (seq < rows)
    ref_slots[okr] = oa.slot_mapping(tables, seq[okr], pos[okr])
    live = ref_slots[ref_slots >= 0]
    assert len(np.unique(live)) == len(live)
    kp = rng.integers(0, 2 ** (8 * nb), size=(NB, Hkv, 16, D), dtype=np.uint64).astype(store)
    vp = rng.integers(0, 2 ** (8 * nb), size=(NB, Hkv, 16, D), dtype=np.uint64).astype(store)
    kn = rng.integers(0, 2 ** (8 * nb), size=(rows, Hkv, D), dtype=np.uint64).astype(store)
    vn = rng.integers(0, 2 ** (8 * nb), size=(rows, Hkv, D), dtype=np.uint64).astype(store)
    log(f"[gpu] append_tokens {dt} D={D} n={rows}")
    dk, dv = to_dev(kp.view(view), dt), to_dev(vp.view(view), dt)
    d_slots = torch.empty(rows, dtype=torch.int64, device="cuda")
    kv.kv_append_tokens(torch.from_numpy(tables).cuda(), torch.from_numpy(seq).cuda(),
                        torch.from_numpy(pos).cuda(), to_dev(kn.view(view), dt),
                        to_dev(vn.view(view), dt), dk, dv, d_slots)
    assert np.array_equal(d_slots.cpu().numpy(), ref_slots)
    ok = ref_slots >= 0
    rk, rv = kp.copy().view(view), vp.copy().view(view)
    oa.reshape_and_cache(kn.view(view)[ok], vn.view(view)[ok], rk, rv, ref_slots[ok])
    assert np.array_equal(bits(to_host(dk, dt)), bits(rk))
    assert np.array_equal(bits(to_host(dv, dt)), bits(rv))


def test_copy_blocks_bit_exact():
    kv = kvlib()
    rng = np.random.default_rng(12)
    L, NB, Hkv, D = 3, 40, 2, 128
    pools = [rng.integers(0, 2 ** 16, size=(NB, Hkv, 16, D), dtype=np.uint64).astype(np.uint16)
             for _ in range(2 * L)]
    perm = rng.permutation(NB)
    pairs = np.stack([perm[:10], perm[10:20]], axis=1).astype(np.int32)  # no chaining
    bad = np.array([[NB + 1, 3], [2, -1]], dtype=np.int32)               # skipped on device
    dev = [to_dev(p, "bf16") for p in pools]
    log("[gpu] copy_blocks")
    kv.kv_copy_blocks(dev[:L], dev[L:], torch.from_numpy(np.concatenate([pairs, bad])).cuda(),
                      NB, Hkv * 16 * D * 2)
    oa.copy_blocks(pools, [tuple(p) for p in pairs])
    for d, p in zip(dev, pools):
        assert np.array_equal(to_host(d, "bf16"), p)


# ---------------------------------------------------------------------------
# the five workloads (+ the copy-on-write variant), end to end
# ---------------------------------------------------------------------------
def run_workload(cfg, S=None, full_pool_compare=True, partition_size=0, block_size=16):
    """One workload through the session's step against the oracle: allocator,
    slots and the written pools bit for bit (pools of the two largest
    workloads on the blocks the step wrote plus a random sample), and every
    output row within tolerance."""
    case = Case(cfg, S=S, partition_size=partition_size, block_size=block_size)
    cows, host_slots, step_pairs = case.device_run()
    sp = case.sp
    # allocator parity (C++ vs oracle model)
    assert len(cows) == len(case.setup_pairs) and [tuple(c) for c in cows] == case.setup_pairs
    assert np.array_equal(host_slots, case.step_slots) and not step_pairs
    assert np.array_equal(case.sess.host_tables[:, :case.tables.shape[1]], case.tables)
    assert np.array_equal(case.sess.host_lens, case.lens)
    # slot mapping kernel and scatter: bit exact
    assert np.array_equal(case.sess.d_slots.cpu().numpy(), case.step_slots)
    if full_pool_compare:
        assert np.array_equal(bits(to_host(case.k_dev, case.kdt)), bits(case.k_ref))
        assert np.array_equal(bits(to_host(case.v_dev, case.kdt)), bits(case.v_ref))
    else:
        blocks = np.unique(np.concatenate([case.step_slots // case.B,
                                           np.random.default_rng(3).integers(0, case.w.num_blocks, 64)]))
        idx = torch.from_numpy(blocks).cuda()
        assert np.array_equal(bits(to_host(case.k_dev[idx], case.kdt)), bits(case.k_ref[blocks]))
        assert np.array_equal(bits(to_host(case.v_dev[idx], case.kdt)), bits(case.v_ref[blocks]))
    got = case.out_dev.cpu().numpy()
    ref = case.oracle_out()
    stats = check_attention(got.reshape(-1, sp.D), ref.reshape(-1, sp.D), case.dt, sp.name)
    log(f"[ok] {sp.name} partition={case.sess.step_partition}: {stats}")
    return case


def test_workload_tiny_fp32():
    run_workload(1)


def test_workload_tiny_fp32_every_partition_size():
    for ps in (16, 32, 48):
        run_workload(1, partition_size=ps)


def test_workload_llama13b_mha_fp16():
    run_workload(2, full_pool_compare=False)


def test_workload_llama70b_gqa_bf16():
    """The benchmark's default workload in the configuration it is timed in:
    16-token blocks, the partition the session chooses (768 tokens), the
    session's placement-ordered plan, cache write fused."""
    case = run_workload(3)
    assert case.sess.step_partition == 768 and case.B == 16 and case.sess.fused
    assert case.sess.d_items is not None and case.sess.shared_tokens == 0


def test_workload_longctx_splitk_bf16():
    run_workload(4, full_pool_compare=False)


def test_workload_prefix_share_bf16():
    case = run_workload(5)
    # 128 shared prefix blocks with reference count 32, read once by the shared-prefix step
    t0 = case.tables[0][:128]
    assert all((case.tables[s][:128] == t0).all() for s in range(case.sp.S))
    assert case.sess.shared_tokens == 2048


def test_workload_prefix_cow_bf16():
    case = run_workload(6)
    assert len(case.setup_pairs) == 31
    assert case.sess.shared_tokens == 2048   # the forked partial block is not common


def test_truncated_workloads_full_output():
    # complete outputs (no sampling) at sizes the oracle finishes quickly
    run_workload(3, S=12)
    run_workload(2, S=3, full_pool_compare=False)


@pytest.mark.parametrize("cfg,S", [(1, None), (2, 3), (3, 16), (6, None)])
def test_fused_and_unfused_steps_are_bitwise_identical(cfg, S):
    """The decode with the cache write fused in gives the same outputs, pools
    and slots, bit for bit, as slot mapping + cache write + decode."""
    case = Case(cfg, S=S)
    res = {}
    for fused in (True, False):
        log(f"[gpu] workload {cfg} fused={fused}")
        case.device_run(fused=fused, shared_prefix=False)
        res[fused] = (case.out_dev.cpu().numpy(), to_host(case.k_dev, case.kdt),
                      to_host(case.v_dev, case.kdt), case.sess.d_slots.cpu().numpy())
    a, b = res[True], res[False]
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))
    assert np.array_equal(bits(a[1]), bits(b[1])) and np.array_equal(bits(a[2]), bits(b[2]))
    assert np.array_equal(a[3], b[3]) and np.array_equal(a[3], case.step_slots)


def test_graph_replay_matches_eager():
    """The fused step captured in a HIP graph: every replay, with eager work
    and synchronisations in between, reproduces the eager outputs, pools and
    slots bit for bit (the captured step holds no memset nodes)."""
    case = Case(3, S=10)
    case.device_run()
    sess, dt = case.sess, case.dt
    eager = (case.out_dev.cpu().numpy().copy(), to_host(case.k_dev, case.kdt).copy(),
             case.sess.d_slots.cpu().numpy().copy())
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
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"[gpu] graph replay {rep}")
        assert np.array_equal(out.cpu().numpy().view(np.uint32), eager[0].view(np.uint32))
        assert np.array_equal(bits(to_host(case.k_dev, case.kdt)), bits(eager[1]))
        assert np.array_equal(sess.d_slots.cpu().numpy(), eager[2])


# ---------------------------------------------------------------------------
# kernel coverage on random ragged shapes (every dtype / head_dim / group)
# ---------------------------------------------------------------------------
def random_case(rng, lens, Hq, Hkv, D, dt, num_blocks=None, poison=True, B=16):
    nbs = [-(-t // B) for t in lens]
    NB = num_blocks or (sum(nbs) + 5)
    perm = rng.permutation(NB)
    tab = np.full((len(lens), max(nbs + [1])), -1, np.int32)
    off = 0
    for s, nb in enumerate(nbs):
        tab[s, :nb] = perm[off:off + nb]
        off += nb
    kp = round_to_dtype(rng.standard_normal((NB, Hkv, B, D)).astype(np.float32), dt)
    vp = round_to_dtype(rng.standard_normal((NB, Hkv, B, D)).astype(np.float32), dt)
    if poison:
        live = np.zeros((NB, B), bool)
        for s, t in enumerate(lens):
            for p in range(t):
                live[tab[s, p // B], p % B] = True
        for pool in (kp, vp):
            b = bits(pool)
            dead = np.argwhere(~live)
            b[dead[:, 0], :, dead[:, 1], :] = POISON[dt]
    q = round_to_dtype(rng.standard_normal((len(lens), Hq, D)).astype(np.float32), dt)
    return q, kp, vp, tab, np.array(lens, np.int32)


def gpu_decode(q, kp, vp, tab, lens, scale, dt, partition_size=0, max_ctx=None, plan=False):
    kv = kvlib()
    S, Hq, D = q.shape
    out = torch.full((S, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    mc = int(lens.max()) if max_ctx is None else max_ctx
    wsb = kv.kv_paged_attention_workspace_bytes(S, Hq, kp.shape[1], D, mc, partition_size)
    ws = torch.full((max(wsb, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda") if wsb else None
    items = None
    if plan:
        items = torch.from_numpy(kv.kv_paged_attention_plan(lens, partition_size)).cuda()
    kv.kv_paged_attention_decode(out, to_dev(q, dt), to_dev(kp, dt), to_dev(vp, dt),
                                 torch.from_numpy(tab).cuda(), torch.from_numpy(lens).cuda(),
                                 scale, mc, ws, partition_size, items)
    torch.cuda.synchronize()
    return out.cpu().numpy()


SHAPES = [(dt, D, G) for dt in ("f32", "f16", "bf16") for D in (64, 128) for G in (1, 2, 4, 8, 16)]


@pytest.mark.parametrize("dt,D,G", SHAPES)
def test_decode_shapes_against_oracle(dt, D, G):
    rng = np.random.default_rng(1000 + SHAPES.index((dt, D, G)))
    lens = [1, 15, 16, 17, 33, 100, 511, 512, 513, 700]
    Hkv = 2
    q, kp, vp, tab, cl = random_case(rng, lens, G * Hkv, Hkv, D, dt)
    scale = float(np.float32(1 / np.sqrt(D)))
    ref = oracle.decode_attention(q, kp, vp, tab, cl, scale, dt)
    for ps, plan in ((0, True), (0, False), (64, True), (16, False)):
        log(f"[gpu] decode {dt} D={D} G={G} partition={ps} plan={plan}")
        got = gpu_decode(q, kp, vp, tab, cl, scale, dt, ps, plan=plan)
        check_attention(got.reshape(-1, D), ref.reshape(-1, D), dt, f"{dt}/{D}/{G}/{ps}/{plan}")


@pytest.mark.parametrize("dt,D,G", [("bf16", 128, 8), ("f16", 128, 2), ("bf16", 128, 16),
                                    ("f32", 64, 4), ("f16", 128, 1), ("bf16", 64, 8)])
def test_decode_append_against_oracle(dt, D, G):
    """Fused cache write + decode on ragged lengths: slots and pools bit exact
    against the oracle's slot formula and scatter, attention within tolerance
    of the oracle run on the scattered pool. The new tokens' slots hold NaN
    beforehand, so a read of the stale slot would show."""
    kv = kvlib()
    rng = np.random.default_rng(2000 + G + D)
    lens = [1, 15, 16, 17, 33, 100, 511, 512, 513, 700, 0]
    Hkv = 2
    q, kp, vp, tab, cl = random_case(rng, lens, G * Hkv, Hkv, D, dt)
    S = len(lens)
    kn = round_to_dtype(rng.standard_normal((S, Hkv, D)).astype(np.float32), dt)
    vn = round_to_dtype(rng.standard_normal((S, Hkv, D)).astype(np.float32), dt)
    seq = np.arange(S, dtype=np.int32)
    ok = cl > 0
    ref_slots = np.full(S, -1, np.int64)
    ref_slots[ok] = oa.slot_mapping(tab, seq[ok], cl[ok] - 1)
    for pool in (kp, vp):  # stale content of the new slots
        b = bits(pool)
        b[ref_slots[ok] // 16, :, ref_slots[ok] % 16, :] = POISON[dt]
    rk, rv = kp.copy(), vp.copy()
    oa.reshape_and_cache(kn[ok], vn[ok], rk, rv, ref_slots[ok])
    scale = float(np.float32(1 / np.sqrt(D)))
    ref = oracle.decode_attention(q, rk, rv, tab, cl, scale, dt)
    for ps, plan in ((0, True), (64, False)):
        log(f"[gpu] decode_append {dt} D={D} G={G} partition={ps} plan={plan}")
        dk, dv = to_dev(kp, dt), to_dev(vp, dt)
        out = torch.full((S, G * Hkv, D), float("nan"), dtype=torch.float32, device="cuda")
        slots = torch.full((S,), 7, dtype=torch.int64, device="cuda")
        mc = int(cl.max())
        wsb = kv.kv_paged_attention_workspace_bytes(S, G * Hkv, Hkv, D, mc, ps)
        ws = torch.full((max(wsb, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda") if wsb else None
        items = torch.from_numpy(kv.kv_paged_attention_plan(cl, ps)).cuda() if plan else None
        kv.kv_paged_attention_decode_append(out, to_dev(q, dt), to_dev(kn, dt), to_dev(vn, dt), dk, dv,
                                            torch.from_numpy(tab).cuda(), torch.from_numpy(cl).cuda(),
                                            scale, mc, slots, ws, ps, items)
        torch.cuda.synchronize()
        assert np.array_equal(slots.cpu().numpy(), ref_slots)
        assert np.array_equal(bits(to_host(dk, dt)), bits(rk))
        assert np.array_equal(bits(to_host(dv, dt)), bits(rv))
        got = out.cpu().numpy()
        assert np.all(got[~ok] == 0.0)
        check_attention(got[ok].reshape(-1, D), ref[ok].reshape(-1, D), dt, f"append {dt}/{D}/{G}/{ps}")


BLOCK_SHAPES = [(B, dt, D, G) for B in (8, 32)
                for dt, D, G in (("bf16", 128, 8), ("f16", 128, 16), ("f32", 64, 2), ("bf16", 128, 1))]


@pytest.mark.parametrize("B,dt,D,G", BLOCK_SHAPES)
def test_block_size_variants_against_oracle(B, dt, D, G):
    """Blocks of 8 and 32 tokens: plain decode, and decode with the fused
    cache write, against the oracle run with the same block size."""
    kv = kvlib()
    rng = np.random.default_rng(3000 + B + G + D)
    lens = [1, 7, 8, 9, 15, 16, 17, 33, 100, 255, 256, 257, 700]
    Hkv = 2
    q, kp, vp, tab, cl = random_case(rng, lens, G * Hkv, Hkv, D, dt, B=B)
    scale = float(np.float32(1 / np.sqrt(D)))
    ref = oracle.decode_attention(q, kp, vp, tab, cl, scale, dt, block_size=B)
    for ps, plan in ((0, True), (64, False), (256, True), (1024, True), (768, False)):
        log(f"[gpu] decode B={B} {dt} D={D} G={G} partition={ps} plan={plan}")
        got = gpu_decode(q, kp, vp, tab, cl, scale, dt, ps, plan=plan)
        check_attention(got.reshape(-1, D), ref.reshape(-1, D), dt, f"B={B} {dt}/{D}/{G}/{ps}")
    # fused cache write of a new token at each sequence's last position
    S = len(lens)
    kn = round_to_dtype(rng.standard_normal((S, Hkv, D)).astype(np.float32), dt)
    vn = round_to_dtype(rng.standard_normal((S, Hkv, D)).astype(np.float32), dt)
    ref_slots = oa.slot_mapping(tab, np.arange(S), cl - 1, block_size=B)
    for pool in (kp, vp):
        bits(pool)[ref_slots // B, :, ref_slots % B, :] = POISON[dt]
    rk, rv = kp.copy(), vp.copy()
    oa.reshape_and_cache(kn, vn, rk, rv, ref_slots, block_size=B)
    ref2 = oracle.decode_attention(q, rk, rv, tab, cl, scale, dt, block_size=B)
    mc = int(cl.max())
    for ps in (0, 1024):  # 1024 tokens: the 700-token sequence's new row is entry 87 (B=8)
        dk, dv = to_dev(kp, dt), to_dev(vp, dt)
        out = torch.full((S, G * Hkv, D), float("nan"), dtype=torch.float32, device="cuda")
        slots = torch.full((S,), 7, dtype=torch.int64, device="cuda")
        wsb = kv.kv_paged_attention_workspace_bytes(S, G * Hkv, Hkv, D, mc, ps)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda") if wsb else None
        items = torch.from_numpy(kv.kv_paged_attention_plan(cl, ps)).cuda()
        log(f"[gpu] decode_append B={B} {dt} D={D} G={G} partition={ps}")
        kv.kv_paged_attention_decode_append(out, to_dev(q, dt), to_dev(kn, dt), to_dev(vn, dt), dk,
                                            dv, torch.from_numpy(tab).cuda(),
                                            torch.from_numpy(cl).cuda(), scale, mc, slots, ws, ps,
                                            items)
        torch.cuda.synchronize()
        assert np.array_equal(slots.cpu().numpy(), ref_slots)
        assert np.array_equal(bits(to_host(dk, dt)), bits(rk))
        assert np.array_equal(bits(to_host(dv, dt)), bits(rv))
        check_attention(out.cpu().numpy().reshape(-1, D), ref2.reshape(-1, D), dt,
                        f"append B={B} partition {ps}")


def test_block_size_workload_llama70b_b32():
    """The 70B-shaped workload (truncated) in 32-token blocks, through the
    session's fused step, against the oracle with the same block size."""
    from gpu_common import Case as _Case  # noqa: F401
    run_workload(3, S=12, block_size=32)


def test_plan_and_padded_grid_are_bitwise_identical():
    rng = np.random.default_rng(40)
    dt, D, Hkv, G = "bf16", 128, 8, 8
    lens = [0, 1, 700, 4097, 512, 33, 1500]
    q, kp, vp, tab, cl = random_case(rng, lens, G * Hkv, Hkv, D, dt)
    for ps in (128, 512):
        a = gpu_decode(q, kp, vp, tab, cl, 0.088, dt, ps, plan=True)
        b = gpu_decode(q, kp, vp, tab, cl, 0.088, dt, ps, plan=False)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        assert np.all(a[0] == 0.0)


def test_zero_length_and_invalid_sequences():
    rng = np.random.default_rng(21)
    dt, D, Hkv, G = "bf16", 128, 2, 4
    lens = [40, 0, 33, 20]
    q, kp, vp, tab, cl = random_case(rng, lens, G * Hkv, Hkv, D, dt)
    tab[2, 1] = 10_000          # live entry outside the pool -> that sequence is NaN
    cl2 = cl.copy()
    cl2[3] = tab.shape[1] * 16 + 1  # longer than its table -> NaN
    log("[gpu] invalid sequences")
    got = gpu_decode(q, kp, vp, tab, cl2, 0.1, dt, 16)
    assert np.all(got[1] == 0.0)
    assert np.isnan(got[2]).all() and np.isnan(got[3]).all()
    ref = oracle.decode_attention(q, kp, vp, tab, cl, 0.1, dt, pairs=[(0, h) for h in range(8)])
    check_attention(got[0], ref[0], dt, "valid neighbour")
    # a length beyond max_context_len is caught too
    got = gpu_decode(q, kp, vp, tab, cl, 0.1, dt, 16, max_ctx=32)
    assert np.isnan(got[0]).all() and np.isnan(got[2]).all() and np.isfinite(got[3]).all()


def test_placement_invariance_bitwise():
    """Same logical cache in two different physical placements: identical bits."""
    rng = np.random.default_rng(31)
    dt, D, Hkv, G = "bf16", 128, 4, 8
    lens = [5, 300, 1030, 77]
    q, kp, vp, tab, cl = random_case(rng, lens, G * Hkv, Hkv, D, dt, poison=False)
    NB = kp.shape[0]
    perm = rng.permutation(NB)            # move physical block b to perm[b]
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    tab2 = np.where(tab >= 0, perm[np.maximum(tab, 0)], -1).astype(np.int32)
    for ps in (0, 128):
        a = gpu_decode(q, kp, vp, tab, cl, 0.09, dt, ps)
        b = gpu_decode(q, kp2, vp2, tab2, cl, 0.09, dt, ps)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_shared_prefix_bitwise_equals_duplicated():
    rng = np.random.default_rng(32)
    dt, D, Hkv, G = "bf16", 128, 2, 4
    pre_blocks, tails = 6, [3, 17, 40]
    nb_t = [-(-t // 16) for t in tails]
    NB = pre_blocks + sum(nb_t)
    kp = round_to_dtype(rng.standard_normal((NB, Hkv, 16, D)).astype(np.float32), dt)
    vp = round_to_dtype(rng.standard_normal((NB, Hkv, 16, D)).astype(np.float32), dt)
    lens = np.array([pre_blocks * 16 + t for t in tails], np.int32)
    shared = np.full((3, pre_blocks + max(nb_t)), -1, np.int32)
    off = pre_blocks
    for s, nb in enumerate(nb_t):
        shared[s, :pre_blocks] = np.arange(pre_blocks)
        shared[s, pre_blocks:pre_blocks + nb] = np.arange(off, off + nb)
        off += nb
    # duplicated: every sequence gets a private copy of the prefix blocks
    kd = np.concatenate([kp] + [kp[:pre_blocks]] * 3)
    vd = np.concatenate([vp] + [vp[:pre_blocks]] * 3)
    dup = shared.copy()
    for s in range(3):
        dup[s, :pre_blocks] = NB + s * pre_blocks + np.arange(pre_blocks)
    q = round_to_dtype(rng.standard_normal((3, G * Hkv, D)).astype(np.float32), dt)
    a = gpu_decode(q, kp, vp, shared, lens, 0.1, dt)
    b = gpu_decode(q, kd, vd, dup, lens, 0.1, dt)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("P", [0, 16])
def test_many_short_sequences(P):
    """3,000 sequences of 1..40 tokens: a grid of 6,000+ single-wave units
    (no merge at the default partition), and at the smallest partition (16
    tokens) up to 3 partitions per sequence merged in 6,000 groups."""
    rng = np.random.default_rng(78)
    dt, D, Hkv, G = "bf16", 128, 2, 4
    lens = list(rng.integers(1, 41, 3000))
    q, kp, vp, tab, cl = random_case(rng, lens, G * Hkv, Hkv, D, dt)
    ref = oracle.decode_attention(q, kp, vp, tab, cl, 0.09, dt)
    for plan in (False, True):
        got = gpu_decode(q, kp, vp, tab, cl, 0.09, dt, P, plan=plan)
        log(f"[gpu] many short P={P} plan={plan}",
            check_attention(got.reshape(-1, D), ref.reshape(-1, D), dt, f"3000 short, P={P}"))


_LONG = {}


def _long_case():
    """One 131,071-token sequence beside a 1-token one (oracle computed once)."""
    if not _LONG:
        rng = np.random.default_rng(77)
        dt, D, Hkv, G = "bf16", 128, 1, 8
        q, kp, vp, tab, cl = random_case(rng, [131071, 1], G * Hkv, Hkv, D, dt, poison=False)
        ref = oracle.decode_attention(q, kp, vp, tab, cl, 1 / np.sqrt(D), dt)
        _LONG.update(case=(q, kp, vp, tab, cl), ref=ref, dt=dt, D=D)
    return _LONG


@pytest.mark.parametrize("P", [512, 1024])
def test_one_very_long_sequence(P):
    """256 (or 128) partitions merged in one group, a table far longer than
    the 64 entries a unit stages, and a tail partition of 511 (1,023) tokens;
    the 1-token sequence beside it is checked on its own scale."""
    c = _long_case()
    q, kp, vp, tab, cl = c["case"]
    dt, D, ref = c["dt"], c["D"], c["ref"]
    got = gpu_decode(q, kp, vp, tab, cl, 1 / np.sqrt(D), dt, P, plan=True)
    for s in range(2):
        log(f"[gpu] long sequence P={P} seq {s}",
            check_attention(got[s].reshape(-1, D), ref[s].reshape(-1, D), dt,
                            f"sequence {s} ({cl[s]} tokens), partition {P}"))


def test_split_and_unsplit_agree_and_runs_are_deterministic():
    rng = np.random.default_rng(33)
    dt, D, Hkv, G = "bf16", 128, 2, 4
    lens = [4097, 2000, 16, 9000]
    q, kp, vp, tab, cl = random_case(rng, lens, G * Hkv, Hkv, D, dt)
    ref = oracle.decode_attention(q, kp, vp, tab, cl, 0.088, dt)
    outs = {}
    for ps in (256, 512, 1024):
        outs[ps] = gpu_decode(q, kp, vp, tab, cl, 0.088, dt, ps)
        check_attention(outs[ps].reshape(-1, D), ref.reshape(-1, D), dt, f"partition {ps}")
    again = gpu_decode(q, kp, vp, tab, cl, 0.088, dt, 512)
    assert np.array_equal(again.view(np.uint32), outs[512].view(np.uint32))


def test_workspace_reuse_gives_identical_results():
    """Repeated calls on one workspace (with and without a plan) give
    bit-identical results: nothing from a previous call leaks into the next."""
    kv = kvlib()
    rng = np.random.default_rng(41)
    dt, D, Hkv, G = "bf16", 128, 4, 4
    lens = np.array([3000, 1, 513, 1024, 777], np.int32)
    q, kp, vp, tab, cl = random_case(rng, list(lens), G * Hkv, Hkv, D, dt)
    S, Hq = len(lens), G * Hkv
    P = 256
    mc = int(lens.max())
    wsb = kv.kv_paged_attention_workspace_bytes(S, Hq, Hkv, D, mc, P)
    ws = torch.full((wsb // 4,), float("nan"), dtype=torch.float32, device="cuda")
    args = (to_dev(q, dt), to_dev(kp, dt), to_dev(vp, dt), torch.from_numpy(tab).cuda(),
            torch.from_numpy(cl).cuda())
    items = torch.from_numpy(kv.kv_paged_attention_plan(cl, P)).cuda()
    outs = []
    for rep in range(3):
        out = torch.full((S, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
        kv.kv_paged_attention_decode(out, *args, 0.088, mc, ws, P, items if rep != 1 else None)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert all(np.array_equal(outs[0].view(np.uint32), o.view(np.uint32)) for o in outs[1:])
    ref = oracle.decode_attention(q, kp, vp, tab, cl, 0.088, dt)
    check_attention(outs[0].reshape(-1, D), ref.reshape(-1, D), dt, "workspace reuse")


def _split_case(seed):
    rng = np.random.default_rng(seed)
    dt, D, Hkv, G = "bf16", 128, 4, 4
    lens = np.array([3000, 1, 513, 1024, 777, 2049], np.int32)
    q, kp, vp, tab, cl = random_case(rng, list(lens), G * Hkv, Hkv, D, dt)
    return dt, D, Hkv, G * Hkv, q, kp, vp, tab, cl


def test_incomplete_plan_does_not_leak_into_the_next_call():
    """A plan that leaves out a partition of a split sequence spoils only that
    sequence's output (NaN here: the missing partials are the workspace's NaN
    fill); the complete sequences of the call are right, and the next call on
    the same workspace, with a full plan or none, is right everywhere."""
    kv = kvlib()
    dt, D, Hkv, Hq, q, kp, vp, tab, cl = _split_case(42)
    S, P, mc = len(cl), 256, int(cl.max())
    wsb = kv.kv_paged_attention_workspace_bytes(S, Hq, Hkv, D, mc, P)
    ws = torch.full((wsb // 4,), float("nan"), dtype=torch.float32, device="cuda")
    args = (to_dev(q, dt), to_dev(kp, dt), to_dev(vp, dt), torch.from_numpy(tab).cuda(),
            torch.from_numpy(cl).cuda())
    plan = kv.kv_paged_attention_plan(cl, P)
    # drop one partition of sequence 0 (12 partitions) and one of sequence 5
    keep = np.ones(len(plan), bool)
    keep[np.flatnonzero(plan[:, 0] == 0)[3]] = False
    keep[np.flatnonzero(plan[:, 0] == 5)[0]] = False
    partial_plan = torch.from_numpy(np.ascontiguousarray(plan[keep])).cuda()
    out = torch.full((S, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    kv.kv_paged_attention_decode(out, *args, 0.088, mc, ws, P, partial_plan)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isnan(got[0]).all() and np.isnan(got[5]).all()   # merged with NaN partials
    ref = oracle.decode_attention(q, kp, vp, tab, cl, 0.088, dt)
    check_attention(got[1:5].reshape(-1, D), ref[1:5].reshape(-1, D), dt, "complete groups")
    for items in (torch.from_numpy(plan).cuda(), None):
        out.fill_(float("nan"))
        kv.kv_paged_attention_decode(out, *args, 0.088, mc, ws, P, items)
        torch.cuda.synchronize()
        check_attention(out.cpu().numpy().reshape(-1, D), ref.reshape(-1, D), dt,
                        f"after an incomplete plan ({'plan' if items is not None else 'grid'})")


def test_graph_replays_and_eager_calls_share_a_workspace():
    """A captured split-K decode (decode and merge kernels) replayed with
    eager calls on the same workspace in between: every replay and every
    eager call gives the same bits."""
    kv = kvlib()
    dt, D, Hkv, Hq, q, kp, vp, tab, cl = _split_case(43)
    S, P, mc = len(cl), 512, int(cl.max())
    wsb = kv.kv_paged_attention_workspace_bytes(S, Hq, Hkv, D, mc, P)
    ws = torch.full((wsb // 4,), float("nan"), dtype=torch.float32, device="cuda")
    args = (to_dev(q, dt), to_dev(kp, dt), to_dev(vp, dt), torch.from_numpy(tab).cuda(),
            torch.from_numpy(cl).cuda())
    items = torch.from_numpy(kv.kv_paged_attention_plan(cl, P)).cuda()
    eager = torch.full((S, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    kv.kv_paged_attention_decode(eager, *args, 0.088, mc, ws, P, items)
    torch.cuda.synchronize()
    want = eager.cpu().numpy()
    ref = oracle.decode_attention(q, kp, vp, tab, cl, 0.088, dt)
    check_attention(want.reshape(-1, D), ref.reshape(-1, D), dt, "eager")
    out = torch.full_like(eager, float("nan"))
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            kv.kv_paged_attention_decode(out, *args, 0.088, mc, ws, P, items,
                                         stream=stream.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"[gpu] decode graph replay {rep}")
        assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))
        if rep % 2 == 0:
            eager.fill_(float("nan"))
            kv.kv_paged_attention_decode(eager, *args, 0.088, mc, ws, P, items)
            torch.cuda.synchronize()
            assert np.array_equal(eager.cpu().numpy().view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("cfg,S", [(3, 12), (5, None), (2, 3)])
def test_load_policies_give_identical_bits(cfg, S):
    """Streaming (non-temporal) and cached K/V loads compute the same bits;
    the session picks cached loads exactly when the pool holds shared blocks."""
    kv = kvlib()
    res = {}
    for policy in (kv.KV_LOADS_STREAM, kv.KV_LOADS_CACHED):
        case = Case(cfg, S=S)
        case.device_run(shared_prefix=False)        # the session's own choice
        chosen = case.sess.load_policy
        assert chosen == (kv.KV_LOADS_CACHED if cfg == 5 else kv.KV_LOADS_STREAM)
        out = torch.full_like(case.out_dev, float("nan"))
        ws = case.sess.workspace
        kv.kv_paged_attention_decode(out, case.q_dev, case.k_dev, case.v_dev, case.sess.d_tables,
                                     case.sess.d_lens, case.sp.scale, case.sess.max_context_len,
                                     ws, case.sess.step_partition, case.sess.d_items,
                                     load_policy=policy)
        torch.cuda.synchronize()
        res[policy] = out.cpu().numpy()
        assert np.array_equal(res[policy].view(np.uint32), case.out_dev.cpu().numpy().view(np.uint32))
        case.sess.close()
    assert np.array_equal(res[0].view(np.uint32), res[1].view(np.uint32))
