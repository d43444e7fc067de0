"""GPU parity of the shared-prefix decode step (kv_paged_attention_decode_append_shared)
against the oracle: attention over every position of every sequence, the shared prefix read
through row 0's table, the tails through each sequence's own table, the new token written
first."""
import numpy as np
import pytest

import oracle
from oracle import attention as oa
from workloads import round_to_dtype
from gpu_common import check_attention, log, to_dev, to_host, bits, POISON

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def kvlib():
    import paged_kv_cache_162_amd as kv
    return kv


def shared_case(rng, S, shared_blocks, tails, Hq, Hkv, D, dt, B=16):
    """S sequences whose first shared_blocks table entries are the same blocks, then tails of
    the given lengths in private blocks; pools shuffled; unused slots poisoned."""
    lens = [shared_blocks * B + t for t in tails]
    tail_nbs = [-(-(t) // B) if t > 0 else 0 for t in tails]
    NB = shared_blocks + sum(tail_nbs) + 7
    perm = rng.permutation(NB)
    shared = perm[:shared_blocks]
    tab = np.full((S, shared_blocks + max(tail_nbs + [1])), -1, np.int32)
    off = shared_blocks
    for s in range(S):
        tab[s, :shared_blocks] = shared
        tab[s, shared_blocks:shared_blocks + tail_nbs[s]] = perm[off:off + tail_nbs[s]]
        off += tail_nbs[s]
    kp = round_to_dtype(rng.standard_normal((NB, Hkv, B, D)).astype(np.float32), dt)
    vp = round_to_dtype(rng.standard_normal((NB, Hkv, B, D)).astype(np.float32), dt)
    live = np.zeros((NB, B), bool)
    for s, t in enumerate(lens):
        for p_ in range(t):
            live[tab[s, p_ // B], p_ % B] = True
    for pool in (kp, vp):
        b = bits(pool)
        dead = np.argwhere(~live)
        b[dead[:, 0], :, dead[:, 1], :] = POISON[dt]
    q = round_to_dtype(rng.standard_normal((S, Hq, D)).astype(np.float32), dt)
    return q, kp, vp, tab, np.array(lens, np.int32)


# (dtype, group, block size, partition, plan): group 1 takes the vector-ALU decode kernel, the
# others the MFMA kernel; a partition below the 700-token tail makes the merge kernel combine
CASES = [("bf16", 8, 16, 0, True), ("bf16", 8, 16, 256, False), ("f16", 4, 16, 128, True),
         ("bf16", 16, 16, 0, True), ("bf16", 8, 8, 0, True), ("bf16", 4, 32, 64, True),
         ("bf16", 1, 16, 0, True), ("f16", 1, 8, 128, False), ("f16", 2, 16, 0, False),
         ("bf16", 6, 16, 0, True), ("f16", 3, 32, 128, False)]


def run_shared_case(rng, dt, G, B, P, plan, S, Hkv, shared_blocks, tails, D=128):
    """One fused shared-prefix step against the oracle: slots, both pools bit for bit, the
    output within the 16-bit tolerance."""
    kv = kvlib()
    q, kp, vp, tab, cl = shared_case(rng, S, shared_blocks, tails, G * Hkv, Hkv, D, dt, B)
    shared = shared_blocks * B
    scale = float(np.float32(1 / np.sqrt(D)))
    kn = round_to_dtype(rng.standard_normal((S, Hkv, D)).astype(np.float32), dt)
    vn = round_to_dtype(rng.standard_normal((S, Hkv, D)).astype(np.float32), dt)
    ref_slots = oa.slot_mapping(tab, np.arange(S), cl - 1, block_size=B)
    for pool in (kp, vp):  # stale content of the new slots
        bits(pool)[ref_slots // B, :, ref_slots % B, :] = POISON[dt]
    rk, rv = kp.copy(), vp.copy()
    oa.reshape_and_cache(kn, vn, rk, rv, ref_slots, block_size=B)
    ref = oracle.decode_attention(q, rk, rv, tab, cl, scale, dt, block_size=B)

    tail_lens = cl - shared
    mt = int(tail_lens.max())
    wsb = kv.kv_paged_attention_workspace_bytes(S, G * Hkv, Hkv, D, mt, P)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda") if wsb else None
    aux = torch.full((kv.kv_paged_attention_shared_aux_bytes(S, G * Hkv, Hkv, D, shared) // 4,), float("nan"),
                     dtype=torch.float32, device="cuda")
    items = torch.from_numpy(kv.kv_paged_attention_plan(tail_lens, P)).cuda() if plan else None
    dk, dv = to_dev(kp, dt), to_dev(vp, dt)
    out = torch.full((S, G * Hkv, D), float("nan"), dtype=torch.float32, device="cuda")
    slots = torch.full((S,), 7, dtype=torch.int64, device="cuda")
    log(f"[gpu] shared prefix {dt} S={S} G={G} Hkv={Hkv} B={B} shared={shared} P={P} plan={plan}")
    kv.kv_paged_attention_decode_append_shared(out, to_dev(q, dt), to_dev(kn, dt), to_dev(vn, dt),
                                               dk, dv, torch.from_numpy(tab).cuda(),
                                               torch.from_numpy(cl).cuda(), scale, shared, mt,
                                               slots, aux, ws, P, items)
    torch.cuda.synchronize()
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    assert np.array_equal(bits(to_host(dk, dt)), bits(rk))
    assert np.array_equal(bits(to_host(dv, dt)), bits(rv))
    log(check_attention(out.cpu().numpy().reshape(-1, D), ref.reshape(-1, D), dt,
                        f"shared {dt} S={S} G={G} B={B} shared={shared} P={P}"))


@pytest.mark.parametrize("dt,G,B,P,plan", CASES)
def test_shared_prefix_step_against_oracle(dt, G, B, P, plan):
    rng = np.random.default_rng(9000 + G + B + P + plan)
    S = 37
    # 664 / 656 / 640 shared positions: two ranges of 8 slices of 64 positions, the second
    # holding 2-3 slices (the last one ragged) and 5-6 waves without keys
    shared_blocks = {8: 83, 16: 41, 32: 20}[B]
    tails = list(rng.integers(1, 300, S))
    tails[0], tails[1], tails[2] = 1, 2, 700       # new token only; tiny; several partitions
    run_shared_case(rng, dt, G, B, P, plan, S, 2, shared_blocks, tails)


# Shapes of the prefix pass's plan: (sequences, group, KV heads, block size, shared blocks).
# 64 x 4 / 8 heads: 16 column tiles per head, 2 ranges of 8 slices of 128; 32 x 4 / 8 heads
# over 8,192 positions: slices of 256, 4 ranges; 2 x 1 / 1 head over 131,072 positions (the
# limit): 16 ranges of 8 slices of 1,024; 3 x 16 / 1 head over 104 positions of 8-token
# blocks: one range of 2 slices, the second 40 positions (a half tile)
PLANS = [(64, 4, 8, 16, 128), (32, 4, 8, 16, 512), (2, 1, 1, 32, 4096), (3, 16, 1, 8, 13)]


@pytest.mark.parametrize("S,G,Hkv,B,shared_blocks", PLANS)
def test_shared_prefix_plans(S, G, Hkv, B, shared_blocks):
    rng = np.random.default_rng(9200 + S + G + shared_blocks)
    tails = list(rng.integers(1, 90, S))
    tails[0] = 1
    run_shared_case(rng, "bf16", G, B, 0, True, S, Hkv, shared_blocks, tails)


def test_shared_prefix_edge_lengths():
    """A sequence of exactly the shared length gets the attention over the shared positions
    and no write; a shorter one gets NaN; the others are unaffected."""
    kv = kvlib()
    rng = np.random.default_rng(9100)
    dt, D, Hkv, G, B = "bf16", 128, 2, 8, 16
    S, shared_blocks = 5, 8
    tails = [5, 9, 1, 30, 17]
    q, kp, vp, tab, cl = shared_case(rng, S, shared_blocks, tails, G * Hkv, Hkv, D, dt, B)
    shared = shared_blocks * B
    cl_run = cl.copy()
    cl_run[1] = shared          # tail 0: prefix only
    cl_run[3] = shared - 3      # shorter than the shared part: invalid
    scale = 0.09
    kn = round_to_dtype(rng.standard_normal((S, Hkv, D)).astype(np.float32), dt)
    vn = round_to_dtype(rng.standard_normal((S, Hkv, D)).astype(np.float32), dt)
    ok = [0, 2, 4]
    ref_slots = oa.slot_mapping(tab[ok], np.arange(len(ok)), cl_run[ok] - 1, block_size=B)
    rk, rv = kp.copy(), vp.copy()
    oa.reshape_and_cache(kn[ok], vn[ok], rk, rv, ref_slots, block_size=B)
    ref = oracle.decode_attention(q[ok], rk, rv, tab[ok], cl_run[ok], scale, dt, block_size=B)
    ref1 = oracle.decode_attention(q[[1]], kp, vp, tab[[1]], cl_run[[1]], scale, dt, block_size=B)
    mt = int(max(cl_run - shared))
    wsb = kv.kv_paged_attention_workspace_bytes(S, G * Hkv, Hkv, D, mt, 0)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda") if wsb else None
    aux = torch.empty(kv.kv_paged_attention_shared_aux_bytes(S, G * Hkv, Hkv, D, shared) // 4,
                      dtype=torch.float32, device="cuda")
    dk, dv = to_dev(kp, dt), to_dev(vp, dt)
    out = torch.full((S, G * Hkv, D), 3.0, dtype=torch.float32, device="cuda")
    slots = torch.full((S,), 7, dtype=torch.int64, device="cuda")
    kv.kv_paged_attention_decode_append_shared(out, to_dev(q, dt), to_dev(kn, dt), to_dev(vn, dt),
                                               dk, dv, torch.from_numpy(tab).cuda(),
                                               torch.from_numpy(cl_run).cuda(), scale, shared,
                                               mt, slots, aux, ws, 0, None)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    sl = slots.cpu().numpy()
    assert np.array_equal(sl[ok], ref_slots) and sl[1] == -1 and sl[3] == -1
    assert np.isnan(got[3]).all()
    check_attention(got[ok].reshape(-1, D), ref.reshape(-1, D), dt, "valid rows")
    check_attention(got[1].reshape(-1, D), ref1.reshape(-1, D), dt, "prefix only")
    assert np.array_equal(bits(to_host(dk, dt)), bits(rk))


@pytest.mark.parametrize("cfg,B", [(5, 16), (6, 16), (5, 8), (5, 32)])
def test_session_shared_step_matches_plain_step(cfg, B):
    """The session's shared-prefix step and its plain fused step on the prefix-sharing
    workloads: identical slots and pools, outputs within the attention tolerance of each other
    and of the oracle."""
    from gpu_common import Case
    res = {}
    for shared in (True, False):
        case = Case(cfg, block_size=B)
        log(f"[gpu] session workload {cfg} B={B} shared_prefix={shared}")
        case.device_run(shared_prefix=shared)
        assert (case.sess.shared_tokens > 0) == shared
        res[shared] = (case.out_dev.cpu().numpy(), to_host(case.k_dev, case.kdt),
                       to_host(case.v_dev, case.kdt), case.sess.d_slots.cpu().numpy())
        case.sess.close()
    a, b = res[True], res[False]
    assert np.array_equal(a[3], b[3]) and np.array_equal(a[3], case.step_slots)
    assert np.array_equal(bits(a[1]), bits(b[1])) and np.array_equal(bits(a[2]), bits(b[2]))
    D = case.sp.D
    check_attention(a[0].reshape(-1, D), b[0].reshape(-1, D), case.dt, "shared vs plain step")
    pairs = [(s, h) for s in range(0, case.sp.S, 5) for h in (0, case.sp.Hq - 1)]
    ref = case.oracle_out(pairs)
    check_attention(np.stack([a[0][s, h] for s, h in pairs]),
                    np.stack([ref[s, h] for s, h in pairs]), case.dt, "shared step vs oracle")


def test_shared_step_graph_replay_matches_eager():
    """The session's shared-prefix step captured in a HIP graph (three launches, no memset
    nodes): every replay, with the outputs, slots and scratch poisoned in between by eager work,
    reproduces the eager step bit for bit."""
    from gpu_common import Case
    case = Case(5)
    case.device_run()
    sess = case.sess
    assert sess.shared_tokens == 2048
    eager = (case.out_dev.cpu().numpy().copy(), to_host(case.k_dev, case.kdt).copy(),
             sess.d_slots.cpu().numpy().copy())
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
        log(f"[gpu] shared step graph replay {rep}")
        assert np.array_equal(out.cpu().numpy().view(np.uint32), eager[0].view(np.uint32))
        assert np.array_equal(bits(to_host(case.k_dev, case.kdt)), bits(eager[1]))
        assert np.array_equal(sess.d_slots.cpu().numpy(), eager[2])
    sess.close()


@pytest.mark.parametrize("where", ["prefix", "tail"])
def test_shared_step_invalid_table_entry(where):
    """An out-of-pool block ID in the shared part of row 0's table makes every output NaN (all
    sequences read the prefix through it); one in a sequence's tail makes only that sequence
    NaN. No load leaves the pool (the kernels read block 0 instead) and the other outputs match
    the oracle."""
    kv = kvlib()
    rng = np.random.default_rng(9200)
    dt, D, Hkv, G, B = "bf16", 128, 2, 8, 16
    S, shared_blocks = 6, 20
    tails = [40, 3, 77, 16, 1, 130]
    q, kp, vp, tab, cl = shared_case(rng, S, shared_blocks, tails, G * Hkv, Hkv, D, dt, B)
    shared = shared_blocks * B
    scale = 0.088
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
    oa.reshape_and_cache(kn, vn, rk, rv, ref_slots, block_size=B)
    ref = oracle.decode_attention(q, rk, rv, tab, cl, scale, dt, block_size=B)
    mt = int(max(cl - shared))
    wsb = kv.kv_paged_attention_workspace_bytes(S, G * Hkv, Hkv, D, mt, 0)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda") if wsb else None
    aux = torch.empty(kv.kv_paged_attention_shared_aux_bytes(S, G * Hkv, Hkv, D, shared) // 4,
                      dtype=torch.float32, device="cuda")
    out = torch.full((S, G * Hkv, D), 3.0, dtype=torch.float32, device="cuda")
    slots = torch.full((S,), 7, dtype=torch.int64, device="cuda")
    log(f"[gpu] shared step, invalid entry in the {where}")
    kv.kv_paged_attention_decode_append_shared(out, to_dev(q, dt), to_dev(kn, dt), to_dev(vn, dt),
                                               to_dev(kp, dt), to_dev(vp, dt),
                                               torch.from_numpy(bad_tab).cuda(),
                                               torch.from_numpy(cl).cuda(), scale, shared, mt,
                                               slots, aux, ws, 0, None)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    if where == "prefix":
        assert np.isnan(got).all()
    else:
        ok = [s for s in range(S) if s != victim]
        assert np.isnan(got[victim]).all()
        check_attention(got[ok].reshape(-1, D), ref[ok].reshape(-1, D), dt, "other sequences")
