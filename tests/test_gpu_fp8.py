"""GPU parity for the fp8 (E4M3) KV cache ("PagedAttention - how vLLM stopped
wasting 80% of your GPU memory", "How does this relate to quantization?").

Bit exact against the oracle: every E4M3 code the device writes (the
elementwise quantiser over every 16-bit input pattern, the cache write, the
fused write). Attention over fp8 pools: within the 16-bit tolerance of the
oracle's float64 attention over the dequantised cache.
"""
import numpy as np
import pytest

import oracle
from oracle import fp8 as ofp8
from workloads import round_to_dtype
from gpu_common import Case, check_attention, log, to_dev, to_host, bits, POISON

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


SCALES = [1.0, 0.25, 0.0123, 3.7, 2.0 ** -20, 1e30]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_quantize_every_16bit_pattern(dt):
    kv = kvlib()
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    host = pats if dt == "bf16" else pats.view(np.float16)
    src = to_dev(host, dt)
    dst = torch.empty(65536, dtype=torch.uint8, device="cuda")
    for scale in SCALES:
        log(f"[gpu] quantize {dt} scale={scale}")
        kv.kv_quantize_fp8(src, dst, scale)
        torch.cuda.synchronize()
        want = ofp8.quantize(host, dt, scale)
        got = dst.cpu().numpy()
        bad = np.nonzero(got != want)[0]
        assert len(bad) == 0, (dt, scale, [(hex(int(pats[i])), hex(got[i]), hex(want[i]))
                                           for i in bad[:8]])


def test_reshape_and_cache_fp8_bit_exact():
    kv = kvlib()
    rng = np.random.default_rng(70)
    NB, Hkv, B, D, n = 12, 4, 16, 128, 40
    kp = rng.integers(0, 256, (NB, Hkv, B, D), dtype=np.uint8)
    vp = rng.integers(0, 256, (NB, Hkv, B, D), dtype=np.uint8)
    slots = rng.permutation(NB * B)[:n].astype(np.int64)
    slots[3], slots[11] = -1, NB * B + 7          # skipped
    for dt in ("bf16", "f16"):
        kn = round_to_dtype(rng.standard_normal((n, Hkv, D)).astype(np.float32) * 3, dt)
        vn = round_to_dtype(rng.standard_normal((n, Hkv, D)).astype(np.float32) * 3, dt)
        dk, dv = to_dev(kp, "e4m3"), to_dev(vp, "e4m3")
        log(f"[gpu] reshape_and_cache_fp8 {dt}")
        kv.kv_reshape_and_cache_fp8(to_dev(kn, dt), to_dev(vn, dt), dk, dv,
                                    torch.from_numpy(slots).cuda(), 0.05, 0.02)
        torch.cuda.synchronize()
        rk, rv = kp.copy(), vp.copy()
        ok = (slots >= 0) & (slots < NB * B)
        ofp8.reshape_and_cache_fp8(kn[ok], vn[ok], rk, rv, slots[ok], dt, 0.05, 0.02)
        assert np.array_equal(dk.cpu().numpy(), rk)
        assert np.array_equal(dv.cpu().numpy(), rv)


def fp8_case(rng, lens, Hq, Hkv, D, dt, B=16, poison=True):
    nbs = [-(-t // B) for t in lens]
    NB = sum(nbs) + 5
    perm = rng.permutation(NB)
    tab = np.full((len(lens), max(nbs + [1])), -1, np.int32)
    off = 0
    for s, nb in enumerate(nbs):
        tab[s, :nb] = perm[off:off + nb]
        off += nb
    # every finite code, subnormals and zeros included
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    kp = rng.choice(finite, (NB, Hkv, B, D))
    vp = rng.choice(finite, (NB, Hkv, B, D))
    if poison:
        live = np.zeros((NB, B), bool)
        for s, t in enumerate(lens):
            for p in range(t):
                live[tab[s, p // B], p % B] = True
        dead = np.argwhere(~live)
        for pool in (kp, vp):
            pool[dead[:, 0], :, dead[:, 1], :] = POISON["e4m3"]
    q = round_to_dtype(rng.standard_normal((len(lens), Hq, D)).astype(np.float32), dt)
    return q, kp, vp, tab, np.array(lens, np.int32)


def gpu_decode_fp8(q, kp, vp, tab, lens, scale, ks, vs, dt, partition_size=0, plan=False):
    kv = kvlib()
    S, Hq, D = q.shape
    out = torch.full((S, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    mc = int(lens.max())
    wsb = kv.kv_paged_attention_workspace_bytes(S, Hq, kp.shape[1], D, mc, partition_size)
    ws = torch.full((max(wsb, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda") if wsb else None
    items = torch.from_numpy(kv.kv_paged_attention_plan(lens, partition_size)).cuda() if plan else None
    kv.kv_paged_attention_decode_fp8(out, to_dev(q, dt), to_dev(kp, "e4m3"), to_dev(vp, "e4m3"),
                                     torch.from_numpy(tab).cuda(), torch.from_numpy(lens).cuda(),
                                     scale, ks, vs, mc, ws, partition_size, items)
    torch.cuda.synchronize()
    return out.cpu().numpy()


SHAPES = [(dt, G, B, D) for D in (128, 64) for dt in ("bf16", "f16") for G in (1, 2, 4, 8, 16)
          for B in (8, 16, 32)]


@pytest.mark.parametrize("dt,G,B,D", SHAPES)
def test_decode_fp8_against_oracle(dt, G, B, D):
    """Head dimension 128 runs the MFMA kernel, 64 the vector-ALU kernel."""
    rng = np.random.default_rng(700 + SHAPES.index((dt, G, B, D)))
    lens = [1, 15, 16, 17, 33, 100, 511, 512, 513, 700]
    Hkv = 2
    q, kp, vp, tab, cl = fp8_case(rng, lens, G * Hkv, Hkv, D, dt, B=B)
    scale, ks, vs = float(np.float32(1 / np.sqrt(D))), 0.07, 0.013
    ref = oracle.decode_attention(q, kp, vp, tab, cl, scale, dt, block_size=B, kv_dtype="e4m3",
                                  k_scale=ks, v_scale=vs)
    for ps, plan in ((0, True), (0, False), (64, True), (32, False)):
        log(f"[gpu] decode fp8 {dt} G={G} B={B} D={D} partition={ps} plan={plan}")
        got = gpu_decode_fp8(q, kp, vp, tab, cl, scale, ks, vs, dt, ps, plan=plan)
        check_attention(got.reshape(-1, D), ref.reshape(-1, D), dt,
                        f"fp8 {dt} G={G} B={B} D={D} ps={ps}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_decode_append_fp8_against_oracle(D, G):
    """The fused step over fp8 pools: each sequence's new token is quantised
    into its last position (pools and slots bit exact against the oracle's
    write), then attention over the updated cache within tolerance."""
    kv = kvlib()
    rng = np.random.default_rng(790 + D + G)
    dt, Hkv, B = "bf16", 2, 16
    lens = [1, 16, 17, 40, 512, 513, 1500]
    q, kp, vp, tab, cl = fp8_case(rng, lens, G * Hkv, Hkv, D, dt, B=B)
    kn = round_to_dtype(rng.standard_normal((len(lens), Hkv, D)).astype(np.float32) * 2, dt)
    vn = round_to_dtype(rng.standard_normal((len(lens), Hkv, D)).astype(np.float32) * 2, dt)
    scale, ks, vs = float(np.float32(1 / np.sqrt(D))), 0.03, 0.011
    slots = oracle.slot_mapping(tab, np.arange(len(lens)), cl - 1, B)
    rk, rv = kp.copy(), vp.copy()
    ofp8.reshape_and_cache_fp8(kn, vn, rk, rv, slots, dt, ks, vs, block_size=B)
    ref = oracle.decode_attention(q, rk, rv, tab, cl, scale, dt, block_size=B, kv_dtype="e4m3",
                                  k_scale=ks, v_scale=vs)
    for ps in (0, 64):
        log(f"[gpu] decode append fp8 D={D} G={G} partition={ps}")
        dk, dv = to_dev(kp, "e4m3"), to_dev(vp, "e4m3")
        S, Hq = q.shape[:2]
        out = torch.full((S, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
        d_slots = torch.full((S,), -7, dtype=torch.int64, device="cuda")
        mc = int(cl.max())
        wsb = kv.kv_paged_attention_workspace_bytes(S, Hq, Hkv, D, mc, ps)
        ws = torch.full((max(wsb, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
        kv.kv_paged_attention_decode_append_fp8(
            out, to_dev(q, dt), to_dev(kn, dt), to_dev(vn, dt), dk, dv,
            torch.from_numpy(tab).cuda(), torch.from_numpy(cl).cuda(), scale, ks, vs, mc,
            d_slots, ws if wsb else None, ps)
        torch.cuda.synchronize()
        assert np.array_equal(d_slots.cpu().numpy(), slots)
        assert np.array_equal(dk.cpu().numpy(), rk)
        assert np.array_equal(dv.cpu().numpy(), rv)
        check_attention(out.cpu().numpy().reshape(-1, D), ref.reshape(-1, D), dt,
                        f"fp8 append D={D} G={G} ps={ps}")


def test_decode_fp8_long_context_split():
    rng = np.random.default_rng(771)
    lens = [4097, 2000, 16, 9000]
    q, kp, vp, tab, cl = fp8_case(rng, lens, 32, 8, 128, "bf16")
    ref = oracle.decode_attention(q, kp, vp, tab, cl, 0.088, "bf16", kv_dtype="e4m3",
                                  k_scale=0.5, v_scale=0.02)
    for ps in (256, 512, 1024):
        log(f"[gpu] decode fp8 long partition={ps}")
        got = gpu_decode_fp8(q, kp, vp, tab, cl, 0.088, 0.5, 0.02, "bf16", ps, plan=True)
        check_attention(got.reshape(-1, 128), ref.reshape(-1, 128), "bf16", f"fp8 long ps={ps}")


def run_fp8_workload(S=None, fused=True):
    case = Case(7, S=S)
    cows, host_slots, _ = case.device_run(fused=fused)
    sp = case.sp
    assert np.array_equal(host_slots, case.step_slots)
    assert np.array_equal(case.sess.d_slots.cpu().numpy(), case.step_slots)
    assert np.array_equal(to_host(case.k_dev, "e4m3"), case.k_ref)
    assert np.array_equal(to_host(case.v_dev, "e4m3"), case.v_ref)
    ref = case.oracle_out()
    stats = check_attention(case.out_dev.cpu().numpy().reshape(-1, sp.D),
                            ref.reshape(-1, sp.D), case.dt, sp.name)
    log(f"[ok] {sp.name} S={sp.S} fused={fused} partition={case.sess.step_partition}: {stats}")
    return case


def test_workload_llama70b_gqa_fp8_cut():
    run_fp8_workload(S=16)


def test_workload_llama70b_gqa_fp8_full():
    run_fp8_workload()


def test_fp8_fused_step_is_bit_identical_to_unfused():
    res = {}
    for fused in (True, False):
        case = run_fp8_workload(S=16, fused=fused)
        res[fused] = (case.out_dev.cpu().numpy(), to_host(case.k_dev, "e4m3"),
                      to_host(case.v_dev, "e4m3"), case.sess.d_slots.cpu().numpy())
    for a, b in zip(res[True], res[False]):
        assert np.array_equal(bits(a) if a.dtype != np.int64 else a,
                              bits(b) if b.dtype != np.int64 else b)



def test_fp8_graph_replay_matches_eager():
    """The fused fp8 step captured in a HIP graph: every replay, with eager
    work and synchronisations in between, reproduces the eager outputs, pools
    and slots bit for bit."""
    case = Case(7, S=10)
    case.device_run()
    sess = case.sess
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
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"[gpu] fp8 graph replay {rep}")
        assert np.array_equal(out.cpu().numpy().view(np.uint32), eager[0].view(np.uint32))
        assert np.array_equal(to_host(case.k_dev, "e4m3"), eager[1])
        assert np.array_equal(to_host(case.v_dev, "e4m3"), eager[2])
        assert np.array_equal(sess.d_slots.cpu().numpy(), eager[3])
