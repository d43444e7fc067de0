"""Pins for the block-manager and size oracles (CPU only).

Golden values come from tests/golden/*.json, each citing the page passage
that prints them. Property tests check the invariants against a model-free
recount.
"""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import BlockManager, KVError
from oracle.block_manager import run_ops
from workloads import make_workload

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# page fixtures
# ---------------------------------------------------------------------------
def test_eight_request_scenario_exact_integers():
    g = gold("eight_requests.json")
    B = g["block_size"]
    assert sum(g["lengths"]) == g["total_tokens"]
    blocks = [oracle.blocks_for_tokens(t, B) for t in g["lengths"]]
    assert blocks == g["blocks"]
    assert [b * B for b in blocks] == g["slots"]
    assert [oracle.waste_slots(t, B) for t in g["lengths"]] == g["wasted"]
    assert sum(blocks) == g["total_blocks"] and sum(blocks) * B == g["total_slots"]
    assert sum(g["wasted"]) == g["total_wasted"]
    assert round(100 * g["total_wasted"] / g["total_slots"], 1) == g["waste_percent_one_decimal"]
    # pool: 24 GB / 8 MB blocks, capacity = blocks * block size
    assert g["cache_gb"] * 1024 // g["block_mb"] == g["pool_blocks"]
    assert B * g["bytes_per_token_kb"] // 1024 == g["block_mb"]
    bm = BlockManager(g["pool_blocks"], B)
    assert bm.capacity_tokens() == g["capacity_tokens"]
    # allocate the eight requests through the manager
    for t in g["lengths"]:
        s = bm.create()
        bm.append(s, t)
    assert bm.num_free() == g["free_after_eight"]
    per = oracle.blocks_for_tokens(g["extra_request_tokens"], B)
    assert per == g["extra_request_blocks"]
    assert bm.num_free() // per == g["extra_requests_admissible"]
    c = g["contiguous"]
    reserved = len(g["lengths"]) * c["max_seq_len"]
    assert round(100 * (reserved - g["total_tokens"]) / reserved, 1) == c["waste_percent_one_decimal"]
    # the page sizes one reservation as 2,048 x 512 KB = 1,048,576 KB and
    # reads that as 1.05 GB (10^6 KB per GB), so 24 GB holds 22 of them
    reservation_kb = c["max_seq_len"] * g["bytes_per_token_kb"]
    assert reservation_kb == 1_048_576 and round(reservation_kb / 1e6, 2) == 1.05
    assert math.floor(g["cache_gb"] * 1e6 / reservation_kb) == c["max_concurrent"]


def test_capacity_exhaustion_is_all_or_nothing():
    g = gold("eight_requests.json")
    bm = BlockManager(g["pool_blocks"], 16)
    s = bm.create()
    bm.append(s, g["capacity_tokens"])          # fills every slot exactly
    assert bm.num_free() == 0
    snap = (list(bm.refcount), list(bm.free), bm.table(s), bm.length(s))
    with pytest.raises(KVError) as e:
        bm.append(s, 1)
    assert e.value.code == "OOM"
    assert snap == (list(bm.refcount), list(bm.free), bm.table(s), bm.length(s))
    t = bm.create()
    with pytest.raises(KVError):
        bm.append(t, 1)
    assert bm.table(t) == [] and bm.length(t) == 0


def test_worked_allocator_trace():
    g = gold("worked_trace.json")
    bm = BlockManager(g["num_blocks"], g["block_size"], free_order=g["free_order"])
    seqs = {}
    for st_ in g["steps"]:
        if st_["op"] == "admit":
            seqs[st_["seq"]] = bm.create()
            _, pairs = bm.append(seqs[st_["seq"]], st_["tokens"])
            assert pairs == []
        elif st_["op"] == "fork":
            seqs[st_["seq"]] = bm.fork(seqs[st_["parent"]])
        elif st_["op"] == "append":
            _, pairs = bm.append(seqs[st_["seq"]], st_["tokens"])
            assert len(pairs) == st_["expect_cow"]
        elif st_["op"] == "finish":
            bm.free_seq(seqs.pop(st_["seq"]))
            assert set(st_["expect_free_contains"]) <= set(bm.free)
        if "expect_table" in st_:
            assert bm.table(seqs[st_["seq"]]) == st_["expect_table"], st_
        for blk, rc in st_.get("expect_refcount", {}).items():
            assert bm.refcount[int(blk)] == rc


def test_token40_layout():
    g = gold("token40.json")
    bm = BlockManager(8, g["block_size"])
    s = bm.create()
    slots, _ = bm.append(s, g["tokens"])
    table = bm.table(s)
    assert len(table) == g["blocks"]
    for i, (a, b) in enumerate(g["ranges"]):
        for p in range(a, b + 1):
            assert slots[p] // g["block_size"] == table[i]


def _sampling_total(parent_retained: bool):
    g = gold("parallel_sampling.json")
    B = g["block_size"]
    bm = BlockManager(4096, B)
    p = bm.create()
    bm.append(p, g["prompt_tokens"])
    assert len(bm.table(p)) == g["page_prompt_blocks"]
    n_children = g["completions"] if parent_retained else g["completions"] - 1
    kids = [bm.fork(p) for _ in range(n_children)]
    writers = kids if parent_retained else [p] + kids
    copies = 0
    for w in writers:
        _, pairs = bm.append(w, g["completion_tokens"])
        copies += len(pairs)
    return 4096 - bm.num_free(), copies


def test_parallel_sampling_accounting():
    g = gold("parallel_sampling.json")
    B = g["block_size"]
    assert oracle.blocks_for_tokens(g["prompt_tokens"], B) == g["page_prompt_blocks"]
    assert oracle.blocks_for_tokens(g["completion_tokens"], B) == g["page_blocks_per_completion"]
    total4, cow4 = _sampling_total(parent_retained=False)
    total5, cow5 = _sampling_total(parent_retained=True)
    assert total4 == g["exact_total_four_holders"] and cow4 == g["completions"] - 1
    assert total5 == g["exact_total_parent_retained"] and cow5 == g["completions"]
    # the page's count is an upper bound on the exact ones
    page = g["page_prompt_blocks"] + g["completions"] * g["page_blocks_per_completion"] \
        + g["page_copied_blocks_upper_bound"]
    assert page == g["page_total_blocks_approx"] and total5 <= page
    assert page * B == g["page_total_slots"]
    assert g["completions"] * (g["prompt_tokens"] + g["completion_tokens"]) == g["unshared_tokens"]
    assert round(100 * (1 - page * B / g["unshared_tokens"])) == g["page_saving_percent_approx"]


def test_kv_size_formula_examples():
    ex = gold("kv_sizes.json")["examples"]
    a = ex[0]
    n = oracle.kv_cache_bytes(a["layers"], a["kv_heads"], a["head_dim"], a["seq_len"], a["bytes"])
    assert n == 1_677_721_600 and round(n / 1e9, 1) == a["approx_gb"]
    assert a["requests"] * n > a["requests_exceed_gb"] * 1e9
    b = ex[1]
    blk = oracle.kv_cache_bytes(b["layers"], b["kv_heads"], b["head_dim"], b["seq_len"], b["bytes"])
    assert blk == b["exact_bytes"]
    rb = blk * b["request_block_layers"] * b["request_block_kv_heads"]
    assert round(rb / 2 ** 20) == b["request_block_approx_mb"]
    c = ex[2]
    assert oracle.kv_cache_bytes(c["layers"], c["kv_heads"], c["head_dim"], c["seq_len"],
                                 c["bytes"]) == c["exact_bytes"]
    d = ex[3]
    assert round(100 * (1 - d["used_tokens"] / d["reserved_tokens"])) == d["waste_percent_int"]


def test_decode_call_bytes_accounts_exact_lengths():
    acc = oracle.decode_call_bytes([5, 16, 17, 40], 4, 4, 64, 4)
    assert acc["kv"] == 78 * 4 * 64 * 4 * 2 == 159_744
    assert acc["tables"] == (1 + 1 + 2 + 3) * 4


# ---------------------------------------------------------------------------
# workload-level accounting (the shapes the GPU runs)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [1, 5, 6])
def test_workload_allocation_counts(cfg):
    w = make_workload(cfg, with_values=False)
    bm = BlockManager(w.num_blocks, free_order=w.free_order)
    h, _, pairs = run_ops(bm, w.setup_ops)
    _, step_slots, step_pairs = run_ops(bm, w.step_ops, h)
    seqs = [h[i] for i in range(w.S)]
    lens = [bm.length(s) for s in seqs]
    assert lens == list(w.context_lens)
    used = w.num_blocks - bm.num_free()
    if cfg == 1:
        assert [len(bm.table(s)) for s in seqs] == [1, 1, 2, 3] and used == 7
    if cfg == 5:
        assert pairs == [] and step_pairs == [] and used == 672
        assert all(bm.refcount[b] == 32 for b in bm.table(seqs[0])[:128])
    if cfg == 6:
        assert len(pairs) == 31 and step_pairs == [] and used == 672
        # the one sequence that wrote last found the partial block unshared
        assert sum(1 for s in seqs if bm.table(s)[128] == bm.table(seqs[0])[128]) >= 1


@pytest.mark.parametrize("cfg", [2, 3])
def test_waste_per_sequence_is_bounded(cfg):
    w = make_workload(cfg, with_values=False)
    waste = [oracle.waste_slots(int(t)) for t in w.context_lens]
    assert min(waste) >= 0 and max(waste) <= 15
    if cfg == 2:  # lengths uniform: mean waste close to 7.5 ("around 8")
        assert 5.0 < np.mean(waste) < 10.0


# ---------------------------------------------------------------------------
# properties under random operation sequences
# ---------------------------------------------------------------------------
ops_strategy = st.lists(
    st.tuples(st.sampled_from(["create", "append", "fork", "free", "swap_out", "swap_in"]),
              st.integers(0, 7), st.integers(0, 40)),
    min_size=1, max_size=60)


@settings(max_examples=200, deadline=None)
@given(ops_strategy)
def test_refcount_conservation(ops):
    NB, B = 24, 4
    bm = BlockManager(NB, B)
    live = []
    for kind, who, n in ops:
        try:
            if kind == "create" or not live:
                live.append(bm.create())
            elif kind == "append":
                s = live[who % len(live)]
                before = (bm.table(s), bm.length(s))
                slots, pairs = bm.append(s, n)
                assert len(slots) == n
                assert len(bm.table(s)) == -(-bm.length(s) // B)
                for p, sl in zip(range(before[1], before[1] + n), slots):
                    assert sl == bm.table(s)[p // B] * B + p % B
                for src, dst in pairs:
                    assert bm.refcount[dst] >= 1 and bm.refcount[src] >= 1
            elif kind == "fork":
                live.append(bm.fork(live[who % len(live)]))
            elif kind == "free":
                bm.free_seq(live.pop(who % len(live)))
            elif kind == "swap_out":
                s = live[who % len(live)]
                t, length = bm.table(s), bm.length(s)
                assert bm.swap_out(s) == t and bm.length(s) == length
            elif kind == "swap_in":
                s = live[who % len(live)]
                ids = bm.swap_in(s)
                assert len(ids) == -(-bm.length(s) // B)
                assert all(bm.refcount[b] == 1 for b in ids)
        except KVError as e:
            assert e.code == "OOM" or (e.code == "STATE" and kind != "create")
        # recount references from the tables; swapped-out sequences hold none
        count = [0] * NB
        for s in live:
            if bm.is_swapped(s):
                continue
            for b in bm.table(s):
                count[b] += 1
        assert count == bm.refcount
        assert sorted(bm.free) == [b for b in range(NB) if count[b] == 0]
        # the last block of a sequence that others share is never written in place
        for s in live:
            if not bm.is_swapped(s):
                assert bm.length(s) <= len(bm.table(s)) * B


def test_errors_change_nothing():
    bm = BlockManager(4, 16)
    s = bm.create()
    bm.append(s, 20)
    with pytest.raises(KVError) as e:
        bm.decref([3])
    assert e.value.code == "STATE"
    with pytest.raises(KVError):
        bm.incref([9])
    with pytest.raises(KVError) as e:
        bm.fork(99)
    assert e.value.code == "STATE"
    t = bm.table(s)
    with pytest.raises(KVError):
        bm.decref(t + t)   # would underflow
    assert bm.table(s) == t and all(bm.refcount[b] == 1 for b in t)
    with pytest.raises(KVError) as e:
        bm.set_free_order([0, 1, 2, 3])
    assert e.value.code == "STATE"


# ---------------------------------------------------------------------------
# swap out / swap in under memory pressure ([3], "The allocation lifecycle";
# [1], "Preemption")
# ---------------------------------------------------------------------------
def _store(bm, seq, slots, tokens, mem):
    for sl, tok in zip(slots, tokens):
        mem[sl] = tok


def _logical(bm, seq, mem):
    B = bm.block_size
    t = bm.table(seq)
    return [mem.get(t[p // B] * B + p % B) for p in range(bm.length(seq))]


def test_swap_round_trip_preserves_logical_contents():
    # A token-addressed model of the pool: slot -> token value. Swapping a
    # sequence out copies its blocks to "host" by table order, the freed blocks
    # are reused by another request, and swapping back in scatters the host
    # copy into the new blocks; the logical token sequence must be unchanged.
    B = 4
    bm = BlockManager(6, B)
    mem = {}
    a = bm.create()
    slots, _ = bm.append(a, 10)                  # 3 blocks, last one half full
    _store(bm, a, slots, [100 + i for i in range(10)], mem)
    before = _logical(bm, a, mem)
    table = bm.swap_out(a)
    assert table == [0, 1, 2] and bm.num_free() == 6 and bm.is_swapped(a)
    host = [[mem.get(b * B + r) for r in range(B)] for b in table]
    # memory pressure: another request takes (and overwrites) the freed blocks
    c = bm.create()
    cs, _ = bm.append(c, 12)
    assert bm.table(c) == [0, 1, 2]              # LIFO: the same blocks, in order
    _store(bm, c, cs, [-1] * 12, mem)
    ids = bm.swap_in(a)
    assert ids == [3, 4, 5] and bm.table(a) == ids
    for b, rows in zip(ids, host):
        for r, tok in enumerate(rows):
            mem[b * B + r] = tok
    assert _logical(bm, a, mem) == before
    # decode can continue: the next token lands in the half-full last block
    s, pairs = bm.append(a, 1)
    assert s == [5 * B + 2] and pairs == []


def test_swap_of_a_forked_sequence_returns_private_blocks():
    bm = BlockManager(8, 4)
    p = bm.create()
    bm.append(p, 6)                               # blocks 0, 1
    c = bm.fork(p)
    assert bm.refcount[:2] == [2, 2]
    assert bm.swap_out(c) == [0, 1]
    assert bm.refcount[:2] == [1, 1] and bm.num_free() == 6   # still held by the parent
    ids = bm.swap_in(c)
    assert ids == [2, 3] and bm.refcount[:4] == [1, 1, 1, 1]
    # the child's half-full last block is private now: no copy-on-write
    _, pairs = bm.append(c, 1)
    assert pairs == []


def test_swap_errors_change_nothing():
    bm = BlockManager(3, 4)
    a = bm.create()
    bm.append(a, 8)                               # blocks 0, 1
    bm.swap_out(a)
    b = bm.create()
    bm.append(b, 9)                               # takes all three blocks
    with pytest.raises(KVError) as e:
        bm.swap_in(a)
    assert e.value.code == "OOM" and bm.is_swapped(a) and bm.num_free() == 0
    for op in (lambda: bm.append(a, 1), lambda: bm.fork(a), lambda: bm.table(a),
               lambda: bm.swap_out(a), lambda: bm.swap_in(b)):
        with pytest.raises(KVError) as e:
            op()
        assert e.value.code == "STATE"
    assert bm.length(a) == 8
    bm.free_seq(a)                                # a swapped-out sequence can be dropped
    with pytest.raises(KVError) as e:
        bm.is_swapped(a)
    assert e.value.code == "STATE"
    bm.free_seq(b)
    assert bm.num_free() == 3 and bm.refcount == [0, 0, 0]


def test_swap_of_an_empty_sequence():
    bm = BlockManager(2, 4)
    a = bm.create()
    assert bm.swap_out(a) == [] and bm.swap_in(a) == []
