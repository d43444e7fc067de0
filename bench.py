"""Benchmark: one decode step of paged attention on one MI355X.

A step is the whole hot path for one layer and one batch: slot mapping of
every sequence's new token, the cache write of its K/V (reshape_and_cache),
and paged decode attention over the whole cache (partition kernel plus, for
sequences longer than one partition, the split-K merge). Inputs are resident
in HBM before the timed region starts. The host block manager's bookkeeping
for the step happens before timing.

Default workload: the Llama-3-70B-shaped grouped-query decode layer, 128
sequences, 64 query / 8 KV heads, head_dim 128, bf16, lognormal lengths
(median 512) - synthetic, seeded data. To measure from HBM rather than the
256 MB last-level cache, the step rotates over several replicas of the pools
and queries (default: enough to exceed 1 GB).

Prints ONE JSON line (see the keys below). `value` is KV GB/s over the step:
the live K and V bytes of every sequence (exact lengths) divided by the step
time.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X published dense bf16 matrix peak


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 500 warm-up steps bring the clocks to their steady state before the
    # 2,000 timed ones (about 130 ms at the 70B-shaped decode step)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", type=int, default=3, help="workload number 1-11")
    ap.add_argument("--partition", type=int, default=0,
                    help="partition tokens (0 = chosen per batch by kv_paged_attention_choose_partition)")
    ap.add_argument("--block-size", type=int, default=16, help="tokens per KV block (8, 16 or 32)")
    ap.add_argument("--replicas", type=int, default=0, help="pool replicas to rotate (0 = auto)")
    ap.add_argument("--prefill-splits", type=int, default=0,
                    help="key runs per prefill block (0 = chosen per step by "
                         "kv_paged_attention_prefill_choose_splits)")
    ap.add_argument("--no-plan", action="store_true", help="padded grid instead of the host work plan")
    ap.add_argument("--no-shared-prefix", action="store_true",
                    help="decode a common prefix per sequence instead of once per batch")
    ap.add_argument("--unfused", action="store_true",
                    help="separate slot-mapping/cache-write launch instead of the fused decode step")
    ap.add_argument("--graph", action="store_true",
                    help="capture each replica's step in a HIP graph and time graph replays")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="time only the chosen workload (the default run also times workloads "
                         "1, 2, 4 and 5 and reports them under per_config)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--pmc-traffic", default="",
                    help="JSON file with the measured HBM traffic per decode call "
                         "(default: profiles/decode_traffic_<workload>.json when it matches the kernels)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="before the timed steps, run kv_copy_blocks over a buffer of known size "
                         "(reference dispatches for scaling the HBM byte counters)")
    ap.add_argument("--pmc-parse", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --copy-calibration` into the traffic JSON and exit")
    ap.add_argument("--pmc-out", default="", help="where --pmc-parse writes its JSON")
    ap.add_argument("--swap", action="store_true",
                    help="measure swap-out / swap-in of one 4096-token sequence of an "
                         "80-layer GQA model (8 KV heads, head_dim 128, bf16) instead")
    return ap.parse_args()


CAL_PAIRS = 4096            # block pairs copied by the calibration dispatch
CAL_BLOCK_BYTES = 32768     # bytes per block and pool (K and V each)


DECODE_SOURCES = ("decode.hip", "decode_kernels.h", "decode_variants.hip", "device_common.h")
PREFILL_SOURCES = ("prefill.hip", "device_common.h")
# a shared-prefix decode step runs the shared-prefix kernel too
SHARED_DECODE_SOURCES = DECODE_SOURCES + ("shared_prefix.hip",)


def kernel_source_digest(sources=DECODE_SOURCES):
    """Digest of the sources the measured kernels are compiled from: measured
    traffic is only reported while the kernels it was taken on are unchanged."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_162_amd", "csrc")
    for name in sources:
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def is_prefill(workload):
    from workloads import spec
    return spec(workload).chunk > 0


def copy_calibration(kv, torch):
    """A plain copy of known size through kv_copy_blocks: CAL_PAIRS blocks of
    CAL_BLOCK_BYTES in each of two pools, i.e. 2*CAL_PAIRS*CAL_BLOCK_BYTES bytes
    read and the same written per dispatch."""
    nb = 2 * CAL_PAIRS
    k = torch.zeros(nb * CAL_BLOCK_BYTES, dtype=torch.uint8, device="cuda")
    v = torch.zeros_like(k)
    pairs = torch.stack([torch.arange(CAL_PAIRS, dtype=torch.int32),
                         torch.arange(CAL_PAIRS, 2 * CAL_PAIRS, dtype=torch.int32)], 1).cuda()
    for _ in range(5):
        kv.kv_copy_blocks([k], [v], pairs, nb, CAL_BLOCK_BYTES)
    torch.cuda.synchronize()
    del k, v


def hbm_read_ceiling(kv, torch, reps=20):
    """Measured HBM read ceiling: kv_hbm_read_probe (non-temporal 16-byte loads,
    the decode kernels' K/V load policy) streaming a 1 GiB buffer, far past the
    256 MB last-level cache; bytes read per second."""
    nbytes = 1 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.random_(0, 256)
    wg = 8192
    sink = torch.empty(wg, dtype=torch.int32, device="cuda")
    for _ in range(3):
        kv.kv_hbm_read_probe(buf, sink, wg)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        kv.kv_hbm_read_probe(buf, sink, wg)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del buf, sink
    return nbytes / (ms * 1e-3) / 1e9


def _counter_rows(d):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return rows


def _mean_counter(rows, kernel_substr, counter):
    """Mean over dispatches of one counter for kernels whose name contains
    kernel_substr (values summed per dispatch first)."""
    per = {}
    for r in rows:
        if kernel_substr in r["Kernel_Name"] and r["Counter_Name"].startswith(counter):
            key = r.get("Dispatch_Id") or r.get("Correlation_Id")
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return (sum(per.values()) / len(per), len(per)) if per else (0.0, 0)


def _max_counter(rows, kernel_substr, counter):
    """Largest per-dispatch value of one counter for kernels whose name
    contains kernel_substr (values summed per dispatch first)."""
    per = {}
    for r in rows:
        if kernel_substr in r["Kernel_Name"] and r["Counter_Name"].startswith(counter):
            key = r.get("Dispatch_Id") or r.get("Correlation_Id")
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return (max(per.values()), len(per)) if per else (0.0, 0)


def pmc_parse(fetch_dir, write_dir, out_path, workload, partition):
    """HBM bytes per decode call from FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for the calibration
    copy, whose true byte count is known. A shared-prefix decode call adds its
    prefix attention (shared_prefix_kernel); a split call its merge launch
    (splitk_merge_kernel, or prefill_merge_kernel for a prefill with key runs)."""
    cal_bytes = 2 * CAL_PAIRS * CAL_BLOCK_BYTES
    prefill = is_prefill(workload)
    res = {"workload": workload, "partition_arg": partition, "calibration_bytes": cal_bytes}
    total = 0.0
    shared = False
    for tag, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _counter_rows(d)
        # the calibration copy is the largest copy_blocks dispatch: a step's own
        # copy-on-write copies run the same kernel on a few blocks
        cal, ncal = _max_counter(rows, "copy_blocks_kernel", counter)
        dec, ndec = _mean_counter(rows, "prefill_mfma" if prefill else "decode_", counter)
        mrg, nmrg = _mean_counter(rows, "prefill_merge" if prefill else "splitk_merge", counter)
        pre, npre = (0.0, 0) if prefill else _mean_counter(rows, "shared_prefix_kernel", counter)
        if ncal == 0 or ndec == 0:
            raise SystemExit(f"{d}: calibration or decode dispatches missing")
        shared = shared or npre > 0
        factor = cal_bytes / (cal * 1024.0)
        per_call = (dec + (mrg if nmrg else 0.0) + (pre if npre else 0.0)) * 1024.0 * factor
        res[tag] = {"counter": counter, "calibration_kib": cal, "factor": factor,
                    "decode_kib": dec, "merge_kib": mrg if nmrg else None,
                    "prefix_kib": pre if npre else None,
                    "decode_dispatches": ndec, "bytes_per_call": per_call}
        total += per_call
    res["kernel_source_digest"] = kernel_source_digest(
        PREFILL_SOURCES if prefill else SHARED_DECODE_SOURCES if shared else DECODE_SOURCES)
    res["bytes_per_launch"] = total
    with open(out_path, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res))


def to_dev(a, dt):
    import torch
    a = np.ascontiguousarray(a)
    if dt == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def kv_bytes(lens, Hkv, D, eb):
    return int(np.sum(lens.astype(np.int64))) * Hkv * D * eb * 2


def decode_alg_bytes(lens, S, Hq, Hkv, D, eb, B=16, kv_eb=None):
    """Algorithmic bytes of one decode-attention call: live K/V (kv_eb bytes
    per element, default eb), queries, fp32 outputs, live block-table entries,
    lengths."""
    nb = int(np.sum((lens.astype(np.int64) + B - 1) // B))
    kv_eb = eb if kv_eb is None else kv_eb
    return kv_bytes(lens, Hkv, D, kv_eb) + S * Hq * D * eb + S * Hq * D * 4 + nb * 4 + S * 4


# The oracle baseline runs in worker processes started fresh (spawn: they never
# touch the GPU); each builds the workload and the oracle's block tables once.
_ORACLE = {}


def _oracle_worker_init(cfg, block_size):
    # one BLAS thread per worker (the parent's limit does not reach a spawned child)
    from threadpoolctl import threadpool_limits
    _ORACLE["blas"] = threadpool_limits(limits=1)
    import oracle
    from oracle.block_manager import run_ops
    from workloads import make_workload
    w = make_workload(cfg, block_size=block_size)
    bm = oracle.BlockManager(w.num_blocks, block_size=block_size, free_order=w.free_order)
    h, _, _ = run_ops(bm, w.setup_ops + w.step_ops)
    tables, lens = bm.packed_tables([h[i] for i in range(w.S)])
    _ORACLE.update(w=w, tables=tables, lens=lens)


def _oracle_worker_run(seqs):
    """The oracle, untouched, for every query head of the sequences `seqs`."""
    import oracle
    w, sp = _ORACLE["w"], _ORACLE["w"].spec
    pairs = [(s, h) for s in seqs for h in range(sp.Hq)]
    kw = dict(kv_dtype=sp.kv_dtype, k_scale=sp.k_scale, v_scale=sp.v_scale) if sp.kv_dtype else {}
    t0 = time.perf_counter()
    oracle.decode_attention(w.q, w.k_pool, w.v_pool, _ORACLE["tables"], _ORACLE["lens"], sp.scale,
                            sp.dtype, block_size=sp.block_size, pairs=pairs, **kw)
    return time.perf_counter() - t0


def host_cores():
    """Cores this process may run on, capped at the 16-core share a one-GPU machine gives."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_baseline(w, seconds):
    """The oracle, untouched, on this host's cores: the whole decode (gather
    through the block table + fp64 attention) of every sequence, split over one
    worker process per core (sequences dealt out longest first to the least
    loaded worker), passes repeated until `seconds` have elapsed (at most 50)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    from threadpoolctl import threadpool_limits
    sp = w.spec
    cores = host_cores()
    lens = w.context_lens.astype(np.int64)
    chunks, load = [[] for _ in range(cores)], np.zeros(cores)
    for s in np.argsort(-lens, kind="stable"):
        c = int(np.argmin(load))
        chunks[c].append(int(s))
        load[c] += lens[s] + 1
    chunks = [c for c in chunks if c]
    passes, t_total = 0, 0.0
    # one BLAS thread per process: the workers are the parallelism
    with threadpool_limits(limits=1):
        # a worker that dies raises here instead of hanging the pool
        with ProcessPoolExecutor(len(chunks), mp_context=mp.get_context("spawn"),
                                 initializer=_oracle_worker_init,
                                 initargs=(sp_cfg(w), sp.block_size)) as pool:
            list(pool.map(_oracle_worker_run, [[c[0]] for c in chunks]))  # warm the workers
            while passes < 50 and (passes == 0 or t_total < seconds):
                t0 = time.perf_counter()
                list(pool.map(_oracle_worker_run, chunks))
                t_total += time.perf_counter() - t0
                passes += 1
    per = t_total / passes
    kvb = kv_bytes(lens, sp.Hkv, sp.D, sp.kv_elem_bytes)
    return {"value": round(kvb / per / 1e9, 4), "unit": "GB/s", "cores": len(chunks),
            "kind": "oracle", "seqs_per_s": round(sp.S / per, 2), "seconds_per_pass": round(per, 3),
            "sample": f"the whole workload ({sp.S} sequences x {sp.Hq} query heads) per pass, "
                      f"{passes} pass(es), sequences split over {len(chunks)} worker processes "
                      f"with one BLAS thread each"}


def sp_cfg(w):
    return w.spec.cfg


MAX_CONTEXT = 8192  # longest context the workloads allow: a contiguous allocator reserves it


def kv_memory(kv, sess, sp, w):
    """Cache memory the host manager holds for the step's sequences: slots in
    held blocks against the tokens they store (paged), and against a
    contiguous reservation of MAX_CONTEXT tokens per sequence. Shared blocks
    count once, so a shared prefix stores more logical tokens than it holds."""
    held_blocks = w.num_blocks - kv.kv_num_free_blocks(sess.pool)
    slots = held_blocks * sp.block_size
    tokens = int(sess.host_lens.astype(np.int64).sum())
    return {"blocks_held": int(held_blocks), "slots_held": int(slots), "tokens": tokens,
            "paged_waste_pct": round(100.0 * (1 - min(tokens, slots) / slots), 2),
            "contiguous_waste_pct": round(100.0 * (1 - tokens / (sp.S * MAX_CONTEXT)), 2),
            "contiguous_reservation_tokens": MAX_CONTEXT,
            "pages_context": "the pages report 60-80% of KV memory wasted by contiguous "
                             "max-length reservation and under 4% with 16-token paging"}


def prefill_flops(lens, counts, Hq, D):
    """Algorithmic flops of the chunked-prefill attention: every chunk row at
    position p takes 2*D multiply-adds for each of its p+1 scores and as many
    for the weighted sum of values, per query head (4*D*(p+1)*Hq flops)."""
    total = 0
    for L, C in zip(lens.tolist(), counts):
        prev = L - C
        total += 4 * Hq * D * (C * prev + C * (C + 1) // 2)
    return total


def prefill_alg_bytes(lens, counts, Hq, Hkv, D, eb, kv_eb, B=16):
    """Algorithmic bytes of one chunked-prefill attention call: every cached
    position's K and V once per sequence (kv_eb bytes per element), the
    queries, the fp32 outputs, the live block-table entries, the lengths and
    the chunk offsets."""
    lens = np.asarray(lens, dtype=np.int64)
    T = int(sum(counts))
    nb = int(np.sum((lens + B - 1) // B))
    S = len(lens)
    return (kv_bytes(lens, Hkv, D, kv_eb) + T * Hq * D * eb + T * Hq * D * 4 + nb * 4
            + S * 4 + (S + 1) * 4)


def prefill_bench(args, w, kv, torch):
    """One step = the chunk's cache write + the causal attention of every chunk
    row (`DecodeSession.prefill_step`), timed like the decode step."""
    from paged_kv_cache_162_amd.session import DecodeSession
    sp = w.spec
    dt = sp.dtype
    kp, vp = to_dev(w.k_pool, sp.cache_dtype), to_dev(w.v_pool, sp.cache_dtype)
    sess = DecodeSession(k_pool=kp, v_pool=vp, num_q_heads=sp.Hq, free_order=w.free_order,
                         use_plan=not args.no_plan, k_scale=sp.k_scale, v_scale=sp.v_scale,
                         prefill_splits=args.prefill_splits or None)
    sess.run_ops(w.setup_ops)
    counts = [sp.chunk] * sp.S
    sess.prepare_prefill(list(range(sp.S)), counts)
    lens = sess.host_lens
    q, kn, vn = to_dev(w.q, dt), to_dev(w.k_new, dt), to_dev(w.v_new, dt)
    T = sp.S * sp.chunk
    out = torch.empty((T, sp.Hq, sp.D), dtype=torch.float32, device="cuda")
    pool_bytes = 2 * kp.numel() * kp.element_size()
    R = args.replicas or max(1, int(np.ceil(1.0e9 / pool_bytes)))
    reps = [(kp, vp, q, kn, vn)] + [(kp.clone(), vp.clone(), q.clone(), kn.clone(), vn.clone())
                                    for _ in range(R - 1)]
    torch.cuda.synchronize()
    if args.copy_calibration:
        copy_calibration(kv, torch)

    def one(k, events=None):
        a, b, qq, kk, vv = reps[k % R]
        sess.prefill_step(qq, kk, vv, out, sp.scale, k_pool=a, v_pool=b, events=events)

    for k in range(args.warmup):
        one(k)
    torch.cuda.synchronize()
    K = args.steps
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for k in range(K):
        one(k)
    t1.record()
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / K
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for k in range(K):
        one(k, ev[k])
    torch.cuda.synchronize()
    att_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    flops = prefill_flops(lens, counts, sp.Hq, sp.D)
    tflops_step = flops / (step_ms * 1e-3) / 1e12
    alg_bytes = prefill_alg_bytes(lens, counts, sp.Hq, sp.Hkv, sp.D, sp.elem_bytes,
                                  sp.kv_elem_bytes, args.block_size)
    # the bound is whichever floor is higher: the algorithmic flops at the
    # dense bf16 matrix peak or the algorithmic bytes at the HBM peak (short
    # chunks over long prefixes do few flops per K/V byte)
    hbm_bound = alg_bytes / (HBM_PEAK_GBS * 1e9) > flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    if hbm_bound:
        achieved, peak, unit = alg_bytes / (att_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = flops / (att_ms * 1e-3) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    traffic = None
    tpath = args.pmc_traffic or os.path.join(ROOT, "profiles", f"prefill_traffic_w{args.workload}.json")
    if os.path.exists(tpath):
        t = json.load(open(tpath))
        if t.get("kernel_source_digest") == kernel_source_digest(PREFILL_SOURCES) and \
                t.get("workload") == args.workload:
            traffic = round(float(t["bytes_per_launch"]))
    res = {
        "metric": "chunked-prefill attention TFLOP/s and query tokens/s, 1 GPU",
        "value": round(tflops_step, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dt, "data": "synthetic",
        "config": {"workload": f"{sp.name}: {sp.description}", "sequences": sp.S,
                   "chunk_tokens": sp.chunk, "q_heads": sp.Hq, "kv_heads": sp.Hkv,
                   "head_dim": sp.D, "block_size": args.block_size,
                   "sum_context": int(lens.sum()), "max_context": int(lens.max()),
                   "flops_per_step": flops, "replicas_rotated": R, "parallelism": "single GPU",
                   "kv_cache_dtype": sp.cache_dtype, "key_runs_per_block": sess.step_splits},
        "query_tokens_per_s": round(T / (step_ms * 1e-3), 1),
        "attention_ms": round(att_ms, 5),
        "roofline": {"bound": "hbm" if hbm_bound else "mfma", "achieved": round(achieved, 2),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": traffic,
                     "kernel": ("kv_paged_attention_prefill_split%s call: prefill_mfma_kernel "
                                "+ prefill_merge_kernel" if sess.step_splits > 1 else
                                "kv_paged_attention_prefill%s call: prefill_mfma_kernel")
                               % ("_fp8" if sp.kv_dtype else ""),
                     "alg_flops_per_launch": flops, "alg_bytes_per_launch": alg_bytes},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = prefill_cpu_baseline(w, lens, counts, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def _prefill_worker_init(cfg, block_size, lens, qs):
    # one BLAS thread per worker, as for the decode baseline
    from threadpoolctl import threadpool_limits
    _ORACLE["blas"] = threadpool_limits(limits=1)
    import oracle
    from oracle.block_manager import run_ops
    from workloads import make_workload
    w = make_workload(cfg, block_size=block_size)
    bm = oracle.BlockManager(w.num_blocks, block_size=block_size, free_order=w.free_order)
    h, _, _ = run_ops(bm, w.setup_ops + w.step_ops)
    tables, _ = bm.packed_tables([h[i] for i in range(w.S)])
    _ORACLE.update(w=w, tables=tables, lens=np.asarray(lens, dtype=np.int32),
                   qs=np.asarray(qs, dtype=np.int32))


def _prefill_worker_run(units):
    """The prefill oracle, untouched, for the chunk rows [r0, r1) of each unit."""
    import oracle
    w, sp = _ORACLE["w"], _ORACLE["w"].spec
    kw = dict(kv_dtype=sp.kv_dtype, k_scale=sp.k_scale, v_scale=sp.v_scale) if sp.kv_dtype else {}
    t0 = time.perf_counter()
    for r0, r1 in units:
        oracle.prefill_attention(w.q, _ORACLE["qs"], w.k_pool, w.v_pool, _ORACLE["tables"],
                                 _ORACLE["lens"], sp.scale, sp.dtype, block_size=sp.block_size,
                                 rows=range(r0, r1), **kw)
    return time.perf_counter() - t0


def prefill_cpu_baseline(w, lens, counts, seconds):
    """The prefill oracle, untouched, on this host's cores: every chunk row of
    the step, in one oracle call per piece of a sequence's chunk - about one
    piece per 512 positions of context, since the oracle's cost per row grows
    with the context and each call also widens the whole query array - the
    pieces dealt out costliest first to one worker process per core, passes
    repeated until `seconds` have elapsed (at most 20)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    from threadpoolctl import threadpool_limits
    sp = w.spec
    qs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    units, cost = [], []
    for s in range(w.S):
        prev, c = int(lens[s]) - int(counts[s]), int(counts[s])
        k = max(1, min(c, int(round(int(lens[s]) / 512))))
        for i in range(k):
            r0, r1 = c * i // k, c * (i + 1) // k
            if r1 > r0:
                units.append((int(qs[s]) + r0, int(qs[s]) + r1))
                cost.append(int(lens[s]) * (r1 - r0))
    cores = host_cores()
    chunks, load = [[] for _ in range(cores)], np.zeros(cores)
    for u in np.argsort(-np.asarray(cost), kind="stable"):
        c = int(np.argmin(load))
        chunks[c].append(units[u])
        load[c] += cost[u]
    chunks = [c for c in chunks if c]
    passes, t_total = 0, 0.0
    with threadpool_limits(limits=1):
        with ProcessPoolExecutor(len(chunks), mp_context=mp.get_context("spawn"),
                                 initializer=_prefill_worker_init,
                                 initargs=(sp_cfg(w), sp.block_size, [int(x) for x in lens],
                                           [int(x) for x in qs])) as pool:
            list(pool.map(_prefill_worker_run, [[c[0]] for c in chunks]))  # warm the workers
            while passes < 20 and (passes == 0 or t_total < seconds):
                t0 = time.perf_counter()
                list(pool.map(_prefill_worker_run, chunks))
                t_total += time.perf_counter() - t0
                passes += 1
    per = t_total / passes
    flops = prefill_flops(lens, counts, sp.Hq, sp.D)
    return {"value": round(flops / per / 1e12, 6), "unit": "TFLOP/s", "cores": len(chunks),
            "kind": "oracle", "seconds_per_pass": round(per, 3), "passes": passes,
            "sample": f"every chunk row of the step ({int(sum(counts))} rows of {w.S} sequences, "
                      f"{len(units)} oracle calls over {len(chunks)} worker processes, one "
                      f"BLAS thread each), {passes} pass(es)"}


def swap_bench(args, kv, torch):
    """Swap bandwidth: one sequence of SWAP_TOKENS tokens of an 80-layer model
    with 8 KV heads of 128 dims in bf16 (the per-layer shape of the 70B-class
    GQA decode workload) goes to pinned host memory and back. The ceiling shown
    beside it is a DMA copy of the same number of contiguous bytes."""
    L, Hkv, B, D, eb = 80, 8, args.block_size, 128, 2
    tokens = SWAP_TOKENS
    nb = -(-tokens // B)
    NB = 2 * nb
    bb = Hkv * B * D * eb
    kp = [torch.empty(NB * bb, dtype=torch.uint8, device="cuda") for _ in range(L)]
    vp = [torch.empty(NB * bb, dtype=torch.uint8, device="cuda") for _ in range(L)]
    for t in kp + vp:
        t.random_(0, 256)
    # scattered like a pool that has seen churn: every other block, shuffled
    g = torch.Generator().manual_seed(162)
    ids = (torch.randperm(NB, generator=g)[:nb].to(torch.int32)).cuda()
    total = nb * L * 2 * bb
    host = torch.empty(total, dtype=torch.uint8, pin_memory=True)
    dev_flat = torch.empty(total, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / reps / 1e3

    reps = max(min(args.steps // 20, 10), 3)
    t_out = timed(lambda: kv.kv_swap_out_blocks(kp, vp, ids, NB, bb, host), reps)
    t_in = timed(lambda: kv.kv_swap_in_blocks(kp, vp, ids, NB, bb, host), reps)
    t_d2h = timed(lambda: host.copy_(dev_flat, non_blocking=True), reps)
    t_h2d = timed(lambda: dev_flat.copy_(host, non_blocking=True), reps)
    # the round trip is bit exact
    kv.kv_swap_out_blocks(kp, vp, ids, NB, bb, host)
    ref = [kp[0][i * bb:(i + 1) * bb].clone() for i in ids[:4].tolist()]
    for t in kp[:1]:
        t.zero_()
    kv.kv_swap_in_blocks(kp, vp, ids, NB, bb, host)
    torch.cuda.synchronize()
    ok = all(torch.equal(r, kp[0][i * bb:(i + 1) * bb]) for r, i in zip(ref, ids[:4].tolist()))
    gbs = lambda t: total / t / 1e9
    print(json.dumps({
        "metric": "swap_bandwidth", "unit": "GB/s", "higher_is_better": True,
        "swap_out": round(gbs(t_out), 2), "swap_in": round(gbs(t_in), 2),
        "dma_copy_d2h": round(gbs(t_d2h), 2), "dma_copy_h2d": round(gbs(t_h2d), 2),
        "swap_out_ms": round(t_out * 1e3, 3), "swap_in_ms": round(t_in * 1e3, 3),
        "bytes": total, "round_trip_bit_exact": ok, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"swap one {tokens}-token sequence, {L} layers x K,V, "
                               f"{Hkv} KV heads x {D} dims, block {B}", "blocks": nb},
    }))


SWAP_TOKENS = 4096


TRAFFIC_NOTE = ("HBM bytes per decode call from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs of "
                "this kernel source, scaled by the counters' reading for a copy of known size "
                "(profiles/decode_traffic_w{w}.json); null when the kernels changed since")
# workloads timed beside the default one, each with its own bench line's numbers
PER_CONFIG = (1, 2, 4, 5)


def run_decode(args, cfg, kv, torch, steps, warmup, primary):
    """Time the decode step on workload `cfg`: K steps back to back over rotating pool
    replicas (inputs resident in HBM), per-call event timing of the attention launches,
    and, for the primary workload, the warm, cache-write and ceiling measurements.
    Returns the numbers of the bench line."""
    from paged_kv_cache_162_amd.session import DecodeSession
    from workloads import make_workload
    w = make_workload(cfg, block_size=args.block_size)
    sp = w.spec
    dt = sp.dtype
    print(f"[bench] workload {sp.name}: S={sp.S} Hq={sp.Hq} Hkv={sp.Hkv} D={sp.D} {dt} "
          f"blocks={w.num_blocks} sum_ctx={int(w.context_lens.sum())} max_ctx={int(w.context_lens.max())}",
          file=sys.stderr, flush=True)
    kp, vp = to_dev(w.k_pool, sp.cache_dtype), to_dev(w.v_pool, sp.cache_dtype)
    sess = DecodeSession(k_pool=kp, v_pool=vp, num_q_heads=sp.Hq, free_order=w.free_order,
                         partition_size=args.partition if primary else 0,
                         use_plan=not args.no_plan, fused=not args.unfused, k_scale=sp.k_scale,
                         v_scale=sp.v_scale, shared_prefix=not args.no_shared_prefix)
    values = {}
    if w.tail_k is not None:
        values = {s: (to_dev(w.tail_k[s], dt), to_dev(w.tail_v[s], dt)) for s in range(sp.S)}
    sess.run_ops(w.setup_ops, values)
    sess.prepare_step(list(range(sp.S)))
    shared = sess.shared_tokens
    memory = kv_memory(kv, sess, sp, w)
    lens = sess.host_lens
    q, kn, vn = to_dev(w.q, dt), to_dev(w.k_new, dt), to_dev(w.v_new, dt)
    out = torch.empty((sp.S, sp.Hq, sp.D), dtype=torch.float32, device="cuda")

    pool_bytes = 2 * kp.numel() * kp.element_size()
    R = (args.replicas if primary else 0) or max(1, int(np.ceil(1.0e9 / pool_bytes)))
    reps = [(kp, vp, q, kn, vn)]
    for _ in range(R - 1):
        reps.append((kp.clone(), vp.clone(), q.clone(), kn.clone(), vn.clone()))
    torch.cuda.synchronize()
    if primary and args.copy_calibration:
        copy_calibration(kv, torch)

    def one(k, events=None):
        a, b, qq, kk, vv = reps[k % R]
        sess.step(qq, kk, vv, out, sp.scale, k_pool=a, v_pool=b, decode_events=events)

    graphs = None
    if primary and args.graph:
        # one graph per replica; the step holds no memset nodes
        for k in range(R):
            one(k)
        torch.cuda.synchronize()
        graphs = []
        cap_stream = torch.cuda.Stream()
        with torch.cuda.stream(cap_stream):
            for k in range(R):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap_stream):
                    one(k)
                graphs.append(g)
        torch.cuda.synchronize()

    def run(k):
        if graphs is not None:
            graphs[k % R].replay()
        else:
            one(k)

    for k in range(warmup):
        run(k)
    torch.cuda.synchronize()
    K = steps
    # timed region: K whole steps back to back, nothing else on the stream
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for k in range(K):
        run(k)
    t_end.record()
    torch.cuda.synchronize()
    step_ms = t_start.elapsed_time(t_end) / K

    # per-call duration of the attention launch(es), events on the launch stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for k in range(K):
        one(k, ev[k])
    torch.cuda.synchronize()
    dec_ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    dec_avg = float(dec_ms.mean())
    # The call's duration for the roofline: when a step is exactly the
    # attention call (fused, no copy-on-write copies) the timed region's
    # average over K back-to-back calls; otherwise the mean of the per-call
    # events, which also time each call apart from its neighbours.
    call_only = not args.unfused and int(sess.d_pairs.shape[0]) == 0
    call_ms = step_ms if call_only else dec_avg

    kvb = kv_bytes(lens, sp.Hkv, sp.D, sp.kv_elem_bytes)
    if shared:
        # the common prefix is read once for the batch, its table entries once
        alg = (decode_alg_bytes(lens - shared, sp.S, sp.Hq, sp.Hkv, sp.D, sp.elem_bytes,
                                args.block_size, sp.kv_elem_bytes)
               + kv_bytes(np.array([shared]), sp.Hkv, sp.D, sp.kv_elem_bytes)
               + shared // args.block_size * 4)
        kv_read = kv_bytes(lens - shared, sp.Hkv, sp.D, sp.kv_elem_bytes) + \
            kv_bytes(np.array([shared]), sp.Hkv, sp.D, sp.kv_elem_bytes)
    else:
        alg = decode_alg_bytes(lens, sp.S, sp.Hq, sp.Hkv, sp.D, sp.elem_bytes, args.block_size,
                               sp.kv_elem_bytes)
        kv_read = kvb
        # a plain step over blocks the batch shares (--no-shared-prefix) reads
        # them once per sequence, mostly from the caches; HBM need hold them once
        common = kv.kv_paged_attention_common_prefix(sess.host_tables, lens, args.block_size)
        if common:
            dup = (sp.S - 1) * (kv_bytes(np.array([common]), sp.Hkv, sp.D, sp.kv_elem_bytes)
                                + common // args.block_size * 4)
            alg -= dup
            kv_read = kv_bytes(lens - common, sp.Hkv, sp.D, sp.kv_elem_bytes) + \
                kv_bytes(np.array([common]), sp.Hkv, sp.D, sp.kv_elem_bytes)
    value = kvb / (step_ms * 1e-3) / 1e9
    res = {
        "workload": f"{sp.name}: {sp.description}", "ms_per_step": round(step_ms, 5),
        "kv_gbs": round(value, 2),
        # bytes the step actually reads: a shared prefix counts once
        "pct_hbm_peak": round(100 * kv_read / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "seqs_per_s": round(sp.S / (step_ms * 1e-3), 1),
        "call_ms": round(call_ms, 5),
        "call_ms_source": ("events over the timed region (the step is the call)" if call_only
                           else "events around each call"),
        "decode_ms": round(dec_avg, 5), "decode_ms_median": round(float(np.median(dec_ms)), 5),
        "partition_tokens": sess.step_partition, "shared_prefix_tokens": shared,
        "steps": K, "warmup": warmup, "replicas_rotated": R,
        "roofline_frac": round(alg / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
    }
    if shared:
        res["logical_kv_gbs"] = round(value, 2)
        res["read_kv_gbs"] = round(kv_read / (step_ms * 1e-3) / 1e9, 2)
    if not primary:
        sess.close()
        return res

    # warm number: same buffers every step
    for k in range(10):
        run(0)
    torch.cuda.synchronize()
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record()
    for k in range(K):
        run(0)
    w1.record()
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / K

    # the step's cache write on its own (the unfused path: slot mapping and
    # write of the S new tokens), events per call
    cw = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for k in range(K):
        a, b, qq, kk, vv = reps[k % R]
        cw[k][0].record()
        sess.write_step_tokens(kk, vv, a, b)
        cw[k][1].record()
    torch.cuda.synchronize()
    cache_write_ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in cw]))
    del reps
    torch.cuda.empty_cache()
    read_gbs = hbm_read_ceiling(kv, torch)

    traffic = None
    tpath = args.pmc_traffic or os.path.join(ROOT, "profiles", f"decode_traffic_w{cfg}.json")
    if os.path.exists(tpath):
        t = json.load(open(tpath))
        sources = SHARED_DECODE_SOURCES if shared else DECODE_SOURCES
        if t.get("kernel_source_digest") == kernel_source_digest(sources) and \
                t.get("workload") == cfg and args.partition == t.get("partition_arg"):
            traffic = round(float(t["bytes_per_launch"]))
    achieved = alg / (call_ms * 1e-3) / 1e9
    res.update({
        "sp": sp, "w": w, "value": value, "kvb": kvb, "memory": memory,
        "warm_ms_per_step": round(warm_ms, 5), "warm_kv_gbs": round(kvb / (warm_ms * 1e-3) / 1e9, 2),
        "cache_write_ms": round(cache_write_ms, 5),
        "decode_kv_gbs": round(kvb / (call_ms * 1e-3) / 1e9, 2),
        "stream_read_gbs": round(read_gbs, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "traffic_source": TRAFFIC_NOTE.format(w=cfg),
                     "kernel": (("kv_paged_attention_decode_append_shared%s call: prefix "
                                 "attention once, then the tails' decode (+ split-K merge) "
                                 "folding it in" if shared else
                                 "kv_paged_attention_decode_append%s call: decode kernel + "
                                 "split-K merge" if not args.unfused else
                                 "kv_paged_attention_decode%s call: decode kernel + split-K merge")
                                % ("_fp8" if sp.kv_dtype else "")),
                     "alg_bytes_per_launch": alg},
    })
    sess.close()
    return res


def main():
    args = parse()
    if args.pmc_parse:
        kind = "prefill" if is_prefill(args.workload) else "decode"
        out = args.pmc_out or os.path.join(ROOT, "profiles", f"{kind}_traffic_w{args.workload}.json")
        pmc_parse(args.pmc_parse[0], args.pmc_parse[1], out, args.workload, args.partition)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1 "
                                   "(the kernels work on one GPU's share of the batch; "
                                   "sharding across GPUs is not implemented)"}))
        sys.exit(2)
    import torch
    from workloads import make_workload
    lib_path = os.path.join(ROOT, "paged_kv_cache_162_amd", "libpagedkv.so")
    if not os.path.exists(lib_path):
        from paged_kv_cache_162_amd import build as b
        b.build()
    import paged_kv_cache_162_amd as kv
    if args.swap:
        swap_bench(args, kv, torch)
        return
    if is_prefill(args.workload):
        prefill_bench(args, make_workload(args.workload, block_size=args.block_size), kv, torch)
        return

    r = run_decode(args, args.workload, kv, torch, args.steps, args.warmup, primary=True)
    sp, w = r.pop("sp"), r.pop("w")
    res = {
        "metric": "paged decode attention KV GB/s (% of HBM peak) and seqs/s per config, 1 GPU",
        "value": round(r["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": sp.dtype,
        "data": "synthetic",
        "config": {
            "workload": r["workload"],
            "sequences": sp.S, "q_heads": sp.Hq, "kv_heads": sp.Hkv, "head_dim": sp.D,
            "block_size": args.block_size, "partition_tokens": r["partition_tokens"],
            "partition_choice": "given" if args.partition else "chosen from the batch's lengths",
            "sum_context": int(w.context_lens.sum()),
            "max_context": int(w.context_lens.max()),
            "kv_bytes_per_step": r["kvb"], "replicas_rotated": r["replicas_rotated"],
            "parallelism": "single GPU", "fused_cache_write": not args.unfused,
            "hip_graph": bool(args.graph), "kv_cache_dtype": sp.cache_dtype,
            "shared_prefix_tokens": r["shared_prefix_tokens"],
        },
        "pct_hbm_peak": r["pct_hbm_peak"],
        "seqs_per_s": r["seqs_per_s"],
        "call_ms": r["call_ms"],
        "call_ms_source": r["call_ms_source"],
        "decode_ms": r["decode_ms"],
        "decode_ms_median": r["decode_ms_median"],
        "decode_kv_gbs": r["decode_kv_gbs"],
        "cache_write_ms": r["cache_write_ms"],
        "stream_read_gbs": r["stream_read_gbs"],
        "warm_ms_per_step": r["warm_ms_per_step"],
        "warm_kv_gbs": r["warm_kv_gbs"],
        "kv_memory": r["memory"],
        "roofline": r["roofline"],
    }
    if "logical_kv_gbs" in r:
        res["logical_kv_gbs"], res["read_kv_gbs"] = r["logical_kv_gbs"], r["read_kv_gbs"]
    if not args.no_per_config and args.workload == 3 and not (args.partition or args.graph
                                                              or args.unfused or args.no_plan):
        per = {"3": {k: r[k] for k in ("workload", "ms_per_step", "kv_gbs", "pct_hbm_peak",
                                          "seqs_per_s", "partition_tokens", "call_ms",
                                          "decode_ms", "roofline_frac", "steps")}}
        for cfg in PER_CONFIG:
            torch.cuda.empty_cache()
            pr = run_decode(args, cfg, kv, torch, min(args.steps, 500), min(args.warmup, 100),
                            primary=False)
            per[str(cfg)] = pr
            print(f"[bench] workload {cfg}: {pr['ms_per_step'] * 1e3:.1f} us per step, "
                  f"{pr['pct_hbm_peak']}% of HBM peak", file=sys.stderr, flush=True)
        res["per_config"] = per
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
