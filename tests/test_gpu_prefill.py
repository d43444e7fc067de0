"""GPU parity for chunked prefill: several query tokens per sequence over the
paged cache, causal within the chunk ("PagedAttention: How vLLM Borrowed
Virtual Memory to Unlock GPU Serving at Scale", "The Successors - SGLang's
RadixAttention and Prefix Sharing" and "Walking Through the Lifecycle",
Prefill).

Attention rows are compared with the oracle's float64 result within the
16-bit tolerance (max |err| / RMS <= 2e-3); the chunk's cache write is bit
exact.
"""
import numpy as np
import pytest

import oracle
from workloads import round_to_dtype, make_workload
from gpu_common import check_attention, log, to_dev, to_host, bits, POISON

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


def prefill_case(rng, prev, chunk, Hq, Hkv, D, dt, B=16, poison=True):
    lens = [p + c for p, c in zip(prev, chunk)]
    nbs = [-(-t // B) for t in lens]
    NB = sum(nbs) + 5
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
        dead = np.argwhere(~live)
        for pool in (kp, vp):
            bits(pool)[dead[:, 0], :, dead[:, 1], :] = POISON[dt]
    q_start = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    q = round_to_dtype(rng.standard_normal((int(q_start[-1]), Hq, D)).astype(np.float32), dt)
    return q, q_start, kp, vp, tab, np.array(lens, np.int32)


def gpu_prefill(q, q_start, kp, vp, tab, lens, scale, dt, plan=True, Hkv=None, max_q=None):
    kv = kvlib()
    T, Hq, D = q.shape
    out = torch.full((T, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    items = None
    if plan:
        it = kv.kv_paged_attention_prefill_plan(q_start, lens, Hq, kp.shape[1])
        items = torch.from_numpy(it).cuda() if len(it) else None
    mq = int(np.diff(q_start).max()) if max_q is None else max_q
    kv.kv_paged_attention_prefill(out, to_dev(q, dt), to_dev(kp, dt), to_dev(vp, dt),
                                  torch.from_numpy(tab).cuda(), torch.from_numpy(lens).cuda(),
                                  torch.from_numpy(q_start).cuda(), scale, mq, items)
    torch.cuda.synchronize()
    return out.cpu().numpy()


SHAPES = [(dt, G, B) for dt in ("bf16", "f16") for G in (1, 2, 3, 8, 16) for B in (8, 16, 32)]


@pytest.mark.parametrize("dt,G,B", SHAPES)
def test_prefill_against_oracle(dt, G, B):
    rng = np.random.default_rng(800 + SHAPES.index((dt, G, B)))
    prev = [0, 5, 16, 100, 700, 33]
    chunk = [1, 16, 17, 40, 100, 0]
    Hkv, D = 2, 128
    q, qs, kp, vp, tab, lens = prefill_case(rng, prev, chunk, G * Hkv, Hkv, D, dt, B=B)
    scale = float(np.float32(1 / np.sqrt(D)))
    ref = oracle.prefill_attention(q, qs, kp, vp, tab, lens, scale, dt, block_size=B)
    for plan in (True, False):
        log(f"[gpu] prefill {dt} G={G} B={B} plan={plan}")
        got = gpu_prefill(q, qs, kp, vp, tab, lens, scale, dt, plan=plan)
        check_attention(got.reshape(-1, D), ref.reshape(-1, D), dt, f"prefill {dt} G={G} B={B}")


def test_prefill_long_prefix_crosses_table_segments():
    # 64 table entries are staged at a time: 3000 cached tokens need several
    rng = np.random.default_rng(880)
    prev, chunk = [3000, 1500], [64, 200]
    q, qs, kp, vp, tab, lens = prefill_case(rng, prev, chunk, 32, 8, 128, "bf16")
    ref = oracle.prefill_attention(q, qs, kp, vp, tab, lens, 0.09, "bf16")
    log("[gpu] prefill long prefix")
    got = gpu_prefill(q, qs, kp, vp, tab, lens, 0.09, "bf16")
    check_attention(got.reshape(-1, 128), ref.reshape(-1, 128), "bf16", "prefill long prefix")


def test_prefill_invalid_sequences_give_nan_rows_only():
    rng = np.random.default_rng(881)
    prev, chunk = [20, 40, 7], [8, 9, 10]
    q, qs, kp, vp, tab, lens = prefill_case(rng, prev, chunk, 16, 2, 128, "bf16")
    tab[1, 1] = kp.shape[0] + 5       # a live entry outside the pool
    lens = lens.copy()
    lens[2] = 5                        # shorter than its chunk of 10
    got = gpu_prefill(q, qs, kp, vp, tab, lens, 0.1, "bf16")
    assert np.isnan(got[qs[1]:qs[2]]).all() and np.isnan(got[qs[2]:qs[3]]).all()
    ref = oracle.prefill_attention(q, qs, kp, vp, tab, lens, 0.1, "bf16", rows=range(qs[0], qs[1]))
    check_attention(got[:qs[1]].reshape(-1, 128), ref[:qs[1]].reshape(-1, 128), "bf16", "valid rows")


def test_prefill_workload_through_the_session():
    """Workload llama70b-gqa-chunked-prefill-bf16 at full size through the
    session: the host manager reserves the chunks, the chunks' K/V are written
    (bit exact on every touched block) and the causal attention runs with the
    host work plan; every output row (all heads) is checked against the oracle."""
    from oracle import attention as oa
    from oracle.block_manager import BlockManager, run_ops
    from paged_kv_cache_162_amd.session import DecodeSession
    w = make_workload(8)
    sp = w.spec
    dt = sp.dtype
    kp_d, vp_d = to_dev(w.k_pool, dt), to_dev(w.v_pool, dt)
    sess = DecodeSession(k_pool=kp_d, v_pool=vp_d, num_q_heads=sp.Hq, free_order=w.free_order)
    sess.run_ops(w.setup_ops)
    counts = [sp.chunk] * sp.S
    host_slots, pairs = sess.prepare_prefill(list(range(sp.S)), counts)
    out = torch.full((sp.S * sp.chunk, sp.Hq, sp.D), float("nan"), dtype=torch.float32,
                     device="cuda")
    log("[gpu] prefill workload step")
    sess.prefill_step(to_dev(w.q, dt), to_dev(w.k_new, dt), to_dev(w.v_new, dt), out, sp.scale)
    torch.cuda.synchronize()
    # oracle side: its own block manager, scatter and attention
    bm = BlockManager(w.num_blocks, free_order=w.free_order)
    h, slots_by_op, _ = run_ops(bm, w.setup_ops + w.step_ops)
    step_slots = np.concatenate([s for s in slots_by_op[len(w.setup_ops):]])
    assert np.array_equal(host_slots, step_slots) and not pairs
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    oa.reshape_and_cache(w.k_new, w.v_new, kp, vp, step_slots)
    tables, lens = bm.packed_tables([h[i] for i in range(sp.S)])
    blocks = np.unique(step_slots // 16)
    idx = torch.from_numpy(blocks).cuda()
    assert np.array_equal(bits(to_host(kp_d[idx], dt)), bits(kp[blocks]))
    assert np.array_equal(bits(to_host(vp_d[idx], dt)), bits(vp[blocks]))
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    qs = np.arange(sp.S + 1, dtype=np.int32) * sp.chunk
    ref = oracle.prefill_attention(w.q, qs, kp, vp, tables, lens, sp.scale, dt)
    check_attention(got.reshape(-1, sp.D), ref.reshape(-1, sp.D), dt, sp.name)
    sess.close()


def test_prefill_graph_replay_matches_eager():
    """The prefill step (cache write + attention) captured in a HIP graph:
    every replay reproduces the eager output and pools bit for bit."""
    from paged_kv_cache_162_amd.session import DecodeSession
    rng = np.random.default_rng(882)
    dt, Hq, Hkv, D, NB = "bf16", 32, 8, 128, 64
    kp = round_to_dtype(rng.standard_normal((NB, Hkv, 16, D)).astype(np.float32), dt)
    vp = round_to_dtype(rng.standard_normal((NB, Hkv, 16, D)).astype(np.float32), dt)
    kd, vd = to_dev(kp, dt), to_dev(vp, dt)
    sess = DecodeSession(k_pool=kd, v_pool=vd, num_q_heads=Hq)
    sess.run_ops([("create", 0), ("append", 0, 100), ("create", 1), ("create", 2),
                  ("append", 2, 33)])
    counts = [40, 17, 64]
    sess.prepare_prefill([0, 1, 2], counts)
    T = sum(counts)
    q = to_dev(round_to_dtype(rng.standard_normal((T, Hq, D)).astype(np.float32), dt), dt)
    kn = to_dev(round_to_dtype(rng.standard_normal((T, Hkv, D)).astype(np.float32), dt), dt)
    vn = to_dev(round_to_dtype(rng.standard_normal((T, Hkv, D)).astype(np.float32), dt), dt)
    out = torch.full((T, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    sess.prefill_step(q, kn, vn, out, 0.088)
    torch.cuda.synchronize()
    eager = (out.cpu().numpy().copy(), to_host(kd, dt).copy(), to_host(vd, dt).copy())
    assert np.isfinite(eager[0]).all()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            sess.prefill_step(q, kn, vn, out, 0.088)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"[gpu] prefill graph replay {rep}")
        assert np.array_equal(out.cpu().numpy().view(np.uint32), eager[0].view(np.uint32))
        assert np.array_equal(bits(to_host(kd, dt)), bits(eager[1]))
        assert np.array_equal(bits(to_host(vd, dt)), bits(eager[2]))
    sess.close()


FP8_SHAPES = [(dt, G, B) for dt in ("bf16", "f16") for G in (1, 8) for B in (8, 16, 32)]


@pytest.mark.parametrize("dt,G,B", FP8_SHAPES)
def test_prefill_fp8_cache_against_oracle(dt, G, B):
    """The prefill kernel over an E4M3 cache: codes widened in LDS, K scale in
    the scores, V scale on the output."""
    kv = kvlib()
    rng = np.random.default_rng(900 + FP8_SHAPES.index((dt, G, B)))
    prev, chunk = [0, 5, 16, 100, 700, 33], [1, 16, 17, 40, 100, 0]
    Hkv, D = 2, 128
    q, qs, _, _, tab, lens = prefill_case(rng, prev, chunk, G * Hkv, Hkv, D, dt, B=B, poison=False)
    NB = int(tab.max()) + 6
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    kp = rng.choice(finite, (NB, Hkv, B, D))
    vp = rng.choice(finite, (NB, Hkv, B, D))
    live = np.zeros((NB, B), bool)
    for s, t in enumerate(lens):
        for p in range(t):
            live[tab[s, p // B], p % B] = True
    dead = np.argwhere(~live)
    for pool in (kp, vp):
        pool[dead[:, 0], :, dead[:, 1], :] = POISON["e4m3"]
    scale, ks, vs = float(np.float32(1 / np.sqrt(D))), 0.06, 0.02
    ref = oracle.prefill_attention(q, qs, kp, vp, tab, lens, scale, dt, block_size=B,
                                   kv_dtype="e4m3", k_scale=ks, v_scale=vs)
    T, Hq = q.shape[0], q.shape[1]
    for plan in (True, False):
        out = torch.full((T, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
        items = None
        if plan:
            items = torch.from_numpy(kv.kv_paged_attention_prefill_plan(qs, lens, Hq, Hkv)).cuda()
        log(f"[gpu] prefill fp8 {dt} G={G} B={B} plan={plan}")
        kv.kv_paged_attention_prefill_fp8(out, to_dev(q, dt), to_dev(kp, "e4m3"), to_dev(vp, "e4m3"),
                                          torch.from_numpy(tab).cuda(), torch.from_numpy(lens).cuda(),
                                          torch.from_numpy(qs).cuda(), scale, ks, vs,
                                          int(np.diff(qs).max()), items)
        torch.cuda.synchronize()
        check_attention(out.cpu().numpy().reshape(-1, D), ref.reshape(-1, D), dt,
                        f"prefill fp8 {dt} G={G} B={B}")


def test_prefill_fp8_session_step():
    """A chunked-prefill step over an fp8 cache through the session: the
    chunk is quantised into the pools (bit exact against the oracle's write)
    and attended causally."""
    from oracle import fp8 as ofp8
    from paged_kv_cache_162_amd.session import DecodeSession
    rng = np.random.default_rng(883)
    dt, Hq, Hkv, D, NB = "bf16", 64, 8, 128, 96
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    kp = rng.choice(finite, (NB, Hkv, 16, D))
    vp = rng.choice(finite, (NB, Hkv, 16, D))
    kd, vd = to_dev(kp, "e4m3"), to_dev(vp, "e4m3")
    sess = DecodeSession(k_pool=kd, v_pool=vd, num_q_heads=Hq, k_scale=0.25, v_scale=0.25)
    ops = [("create", 0), ("append", 0, 300), ("create", 1), ("append", 1, 17), ("create", 2)]
    sess.run_ops(ops)
    counts = [64, 40, 33]
    host_slots, _ = sess.prepare_prefill([0, 1, 2], counts)
    T = sum(counts)
    q = round_to_dtype(rng.standard_normal((T, Hq, D)).astype(np.float32), dt)
    kn = round_to_dtype(rng.standard_normal((T, Hkv, D)).astype(np.float32), dt)
    vn = round_to_dtype(rng.standard_normal((T, Hkv, D)).astype(np.float32), dt)
    out = torch.full((T, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    sess.prefill_step(to_dev(q, dt), to_dev(kn, dt), to_dev(vn, dt), out, 0.088)
    torch.cuda.synchronize()
    rk, rv = kp.copy(), vp.copy()
    ofp8.reshape_and_cache_fp8(kn, vn, rk, rv, host_slots, dt, 0.25, 0.25)
    assert np.array_equal(to_host(kd, "e4m3"), rk) and np.array_equal(to_host(vd, "e4m3"), rv)
    qs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    ref = oracle.prefill_attention(q, qs, rk, rv, sess.host_tables, sess.host_lens, 0.088, dt,
                                   kv_dtype="e4m3", k_scale=0.25, v_scale=0.25)
    check_attention(out.cpu().numpy().reshape(-1, D), ref.reshape(-1, D), dt, "fp8 prefill step")
    sess.close()
