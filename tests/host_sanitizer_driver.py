"""Drives a host-only build of the library (the block manager and the work
planners, compiled with g++ under AddressSanitizer and UndefinedBehaviorSanitizer)
through seeded random operation sequences, checking every result against the
oracle's block manager, then through the planners and step-policy functions on
random inputs. Run by tests/test_host_sanitizers.py in a child process with the
sanitizer runtime preloaded: any memory error or undefined behaviour aborts it.

usage: python host_sanitizer_driver.py <library> <sequences> <seed>
"""
import ctypes as C
import math
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import oracle  # noqa: E402

i32, i64, vp = C.c_int32, C.c_int64, C.c_void_p
P_i32, P_i64 = C.POINTER(i32), C.POINTER(i64)


class Config(C.Structure):
    _fields_ = [("num_blocks", i32), ("block_size", i32), ("num_layers", i32),
                ("num_kv_heads", i32), ("head_dim", i32), ("dtype", C.c_int)]


SIGS = {
    "kv_pool_create": (C.c_int, [C.POINTER(Config), C.POINTER(vp)]),
    "kv_pool_destroy": (None, [vp]),
    "kv_pool_set_free_order": (C.c_int, [vp, i32, P_i32]),
    "kv_num_free_blocks": (i32, [vp]),
    "kv_block_alloc": (C.c_int, [vp, i32, P_i32]),
    "kv_block_incref": (C.c_int, [vp, i32, P_i32]),
    "kv_block_free": (C.c_int, [vp, i32, P_i32]),
    "kv_block_refcount": (i32, [vp, i32]),
    "kv_seq_create": (C.c_int, [vp, P_i64]),
    "kv_seq_fork": (C.c_int, [vp, i64, P_i64]),
    "kv_seq_append": (C.c_int, [vp, i64, i32, P_i64, P_i32, P_i32, P_i32]),
    "kv_seq_free": (C.c_int, [vp, i64]),
    "kv_seq_block_table": (C.c_int, [vp, i64, i32, P_i32, P_i32]),
    "kv_seq_len": (i32, [vp, i64]),
    "kv_seq_pack_tables": (C.c_int, [vp, i32, P_i64, i32, P_i32, P_i32]),
    "kv_seq_swap_out": (C.c_int, [vp, i64, i32, P_i32, P_i32]),
    "kv_seq_swap_in": (C.c_int, [vp, i64, i32, P_i32, P_i32]),
    "kv_seq_is_swapped": (i32, [vp, i64]),
    "kv_pool_shared_blocks": (i32, [vp]),
    "kv_paged_attention_plan": (C.c_int, [P_i32, i32, i32, i32, i32, P_i32, i32, P_i32]),
    "kv_paged_attention_prefill_plan": (C.c_int, [P_i32, P_i32, i32, i32, i32, P_i32, i32, P_i32]),
    "kv_paged_attention_choose_partition": (i32, [P_i32, i32, i32, i32, i32]),
    "kv_paged_attention_common_prefix": (i32, [P_i32, i32, i32, P_i32, i32]),
    "kv_paged_attention_choose_shared_prefix": (i32, [P_i32, i32, i32, P_i32, i32, i32, i32, i32,
                                                      C.c_int]),
    "kv_paged_attention_choose_load_policy": (C.c_int, [vp, i32]),
    "kv_paged_attention_prefill_choose_splits": (i32, [P_i32, P_i32, i32, i32, i32, i32]),
}
STATUS = {0: None, -1: "INVALID", -2: "OOM", -3: "UNSUPPORTED", -5: "STATE"}


def load(path):
    lib = C.CDLL(path)
    for name, (res, args) in SIGS.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


def p32(a):
    return a.ctypes.data_as(P_i32)


def ids_call(fn, pool, seq, cap):
    out = np.zeros(max(cap, 1), np.int32)
    n = i32()
    st = fn(pool, seq, len(out), p32(out), C.byref(n))
    return STATUS[st], out[:n.value].tolist()


def random_sequences(lib, n_seq, rng):
    """Random create/append/fork/free/alloc/incref/decref/swap scripts; after every
    operation the error code, the returned blocks and slots, every reference count,
    the free count and every live table must equal the oracle's."""
    ops = 0
    for _ in range(n_seq):
        NB, B = int(rng.integers(4, 40)), int(rng.choice([4, 8, 16]))
        order = rng.permutation(NB).astype(np.int32)
        cfg = Config(NB, B, 1, 1, 8, 0)
        pool = vp()
        assert lib.kv_pool_create(C.byref(cfg), C.byref(pool)) == 0
        assert lib.kv_pool_set_free_order(pool, NB, p32(order)) == 0
        bm = oracle.BlockManager(NB, B, free_order=order)
        live = []  # (oracle handle, library handle)
        for _ in range(int(rng.integers(1, 80))):
            kind = rng.choice(["create", "append", "append", "fork", "free", "alloc", "incref",
                               "decref", "swap_out", "swap_in"])
            who, n = int(rng.integers(0, 10)), int(rng.integers(0, 3 * B + 2))
            if not live and kind in ("append", "fork", "free", "swap_out", "swap_in"):
                kind = "create"
            ores = cres = oerr = cerr = None
            target = live[who % len(live)] if live else None
            try:
                if kind == "create":
                    ores = bm.create()
                elif kind == "append":
                    ores = bm.append(target[0], n)
                elif kind == "fork":
                    ores = bm.fork(target[0])
                elif kind == "free":
                    bm.free_seq(target[0])
                elif kind == "alloc":
                    ores = bm.alloc(n % 5)
                elif kind == "incref":
                    bm.incref([who % NB])
                elif kind == "decref":
                    bm.decref([who % NB])
                elif kind == "swap_out":
                    ores = bm.swap_out(target[0])
                elif kind == "swap_in":
                    ores = bm.swap_in(target[0])
            except oracle.KVError as e:
                oerr = e.code
            if kind in ("create", "fork"):
                h = i64()
                st = (lib.kv_seq_create(pool, C.byref(h)) if kind == "create"
                      else lib.kv_seq_fork(pool, target[1], C.byref(h)))
                cerr, cres = STATUS[st], h.value
            elif kind == "append":
                slots = np.zeros(max(n, 1), np.int64)
                src, dst, nc = i32(), i32(), i32()
                cerr = STATUS[lib.kv_seq_append(pool, target[1], n, slots.ctypes.data_as(P_i64),
                                                C.byref(src), C.byref(dst), C.byref(nc))]
                cres = (slots[:n].tolist(), [(src.value, dst.value)] if nc.value else [])
            elif kind == "free":
                cerr = STATUS[lib.kv_seq_free(pool, target[1])]
            elif kind == "alloc":
                out = np.zeros(max(n % 5, 1), np.int32)
                cerr = STATUS[lib.kv_block_alloc(pool, n % 5, p32(out))]
                cres = out[:n % 5].tolist()
            elif kind in ("incref", "decref"):
                one = np.array([who % NB], np.int32)
                fn = lib.kv_block_incref if kind == "incref" else lib.kv_block_free
                cerr = STATUS[fn(pool, 1, p32(one))]
            else:
                fn = lib.kv_seq_swap_out if kind == "swap_out" else lib.kv_seq_swap_in
                cerr, cres = ids_call(fn, pool, target[1], lib.kv_seq_len(pool, target[1]) + 1)
            assert oerr == cerr, (kind, oerr, cerr)
            if oerr is None:
                if kind in ("create", "fork"):
                    live.append((ores, cres))
                elif kind == "free":
                    live.remove(target)
                elif kind == "append":
                    assert (list(ores[0]), [tuple(p) for p in ores[1]]) == cres, kind
                elif kind in ("alloc", "swap_out", "swap_in"):
                    assert list(ores) == cres, kind
            assert [lib.kv_block_refcount(pool, b) for b in range(NB)] == bm.refcount
            assert lib.kv_num_free_blocks(pool) == bm.num_free()
            assert lib.kv_pool_shared_blocks(pool) == sum(r > 1 for r in bm.refcount)
            for oh, ch in live:
                assert lib.kv_seq_len(pool, ch) == bm.length(oh)
                assert lib.kv_seq_is_swapped(pool, ch) == int(bm.is_swapped(oh))
                if not bm.is_swapped(oh):
                    st, tab = ids_call(lib.kv_seq_block_table, pool, ch, bm.length(oh) + 1)
                    assert st is None and tab == bm.table(oh)
            ops += 1
        resident = [(oh, ch) for oh, ch in live if not bm.is_swapped(oh)]
        if resident:
            width = max(len(bm.table(oh)) for oh, _ in resident) + 1
            hs = np.array([ch for _, ch in resident], np.int64)
            tab = np.zeros((len(hs), width), np.int32)
            lens = np.zeros(len(hs), np.int32)
            assert lib.kv_seq_pack_tables(pool, len(hs), hs.ctypes.data_as(P_i64), width,
                                          p32(tab), p32(lens)) == 0
            ot, ol = bm.packed_tables([oh for oh, _ in resident], width)
            assert np.array_equal(tab, ot) and np.array_equal(lens, ol)
            lib.kv_paged_attention_choose_load_policy(pool, int(rng.integers(0, 64)))
        lib.kv_pool_destroy(pool)
    return ops


def planners(lib, rounds, rng):
    """The decode and prefill plans list every item once; the choosers return
    values from their documented sets."""
    for _ in range(rounds):
        S = int(rng.integers(0, 60))
        lens = rng.integers(-3, 5000, S).astype(np.int32)
        P = int(rng.choice([16, 128, 512, 768, 1024]))
        hkv, cus = int(rng.integers(1, 41)), int(rng.choice([0, 8, 80, 256]))
        n = i32()
        lib.kv_paged_attention_plan(p32(lens), S, P, hkv, cus, None, 0, C.byref(n))
        items = np.zeros((max(n.value, 1), 2), np.int32)
        assert lib.kv_paged_attention_plan(p32(lens), S, P, hkv, cus, p32(items), n.value,
                                           C.byref(n)) == 0
        want = sorted((s, p) for s in range(S)
                      for p in range(max(1, math.ceil(max(int(lens[s]), 0) / P))))
        assert sorted(map(tuple, items[:n.value].tolist())) == want
        counts = rng.integers(0, 300, S)
        qs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        plen = (lens.astype(np.int64) + counts).clip(0, 2 ** 30).astype(np.int32)
        lib.kv_paged_attention_prefill_plan(p32(qs), p32(plen), S, 64, 8, None, 0, C.byref(n))
        items = np.zeros((max(n.value, 1), 2), np.int32)
        assert lib.kv_paged_attention_prefill_plan(p32(qs), p32(plen), S, 64, 8, p32(items),
                                                   n.value, C.byref(n)) == 0
        hq = int(rng.choice([8, 32, 64, 128]))
        splits = lib.kv_paged_attention_prefill_choose_splits(p32(qs), p32(plen), S, hq, 8,
                                                              int(rng.choice([0, 64, 512])))
        assert 1 <= splits <= 64
        assert lib.kv_paged_attention_choose_partition(p32(lens), S, hkv, 16, 1500) in (512, 768,
                                                                                        1024)
        if S:
            width = int(rng.integers(1, 40))
            tab = rng.integers(0, 4, (S, width)).astype(np.int32)
            tab[:, :width // 2] = tab[0, :width // 2]
            sh = lib.kv_paged_attention_common_prefix(p32(tab), S, width, p32(lens), 16)
            assert 0 <= sh <= width * 16 and sh % 16 == 0
            for dt in (2, 3):   # bf16 and an fp8 cache
                got = lib.kv_paged_attention_choose_shared_prefix(p32(tab), S, width, p32(lens),
                                                                  16, 32, 8, 128, dt)
                assert got == 0 or (got == sh and got >= 256)


if __name__ == "__main__":
    lib = load(sys.argv[1])
    rng = np.random.default_rng(int(sys.argv[3]))
    ops = random_sequences(lib, int(sys.argv[2]), rng)
    planners(lib, 200, rng)
    print(f"ok: {ops} manager operations and 200 planner rounds checked", flush=True)
