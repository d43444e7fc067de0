"""Shared helpers for the GPU parity tests.

A Case builds one workload twice from the same seeded inputs: the oracle side
(pure-Python block manager + numpy scatter/copy, fp64 attention) and the
device side (C ABI block manager + HIP kernels). Nothing computed by the
device is fed to the oracle.
"""
from __future__ import annotations

import sys
from typing import Dict, List, Optional, Tuple

import numpy as np

import oracle
from oracle import attention as oa
from oracle import fp8 as ofp8
from oracle.block_manager import BlockManager
from workloads import make_workload, NP_STORAGE

# a distinctive quiet-NaN payload for poisoned slots
POISON = {"f32": np.uint32(0x7FC0DEAD), "f16": np.uint16(0x7E5A), "bf16": np.uint16(0x7FDA),
          "e4m3": np.uint8(0x7F)}
TOL_FP32_ABS = 1e-5      # fp32 inputs: max |gpu - oracle|
TOL_16BIT_REL_RMS = 2e-3  # 16-bit inputs: max |gpu - oracle| / rms(oracle)


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_dtype(dt: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]


def to_dev(a: np.ndarray, dt: str):
    import torch
    a = np.ascontiguousarray(a)
    if dt == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def to_host(t, dt: str) -> np.ndarray:
    import torch
    t = t.detach().cpu().contiguous()
    if dt == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(a: np.ndarray) -> np.ndarray:
    return a.view({1: np.uint8, 2: np.uint16, 4: np.uint32}[a.dtype.itemsize])


def poison_slots(pool: np.ndarray, dt: str, block_ids, offsets) -> None:
    b = bits(pool)
    b[np.asarray(block_ids), :, np.asarray(offsets), :] = POISON[dt]


def check_attention(got: np.ndarray, ref: np.ndarray, dt: str, what: str) -> dict:
    """Tolerance check: fp32 inputs max abs <= 1e-5; 16-bit inputs
    max abs error / RMS(oracle) <= 2e-3. Both arrays are [n, D] (finite ref)."""
    assert np.isfinite(ref).all(), f"{what}: oracle has non-finite values"
    assert np.isfinite(got).all(), f"{what}: GPU output has non-finite values"
    err = np.abs(got.astype(np.float64) - ref)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    stats = {"max_abs": float(err.max()), "rms": rms, "max_rel_rms": float(err.max() / rms),
             "rms_err_rel": float(np.sqrt(np.mean(err ** 2)) / rms)}
    if dt == "f32":
        assert stats["max_abs"] <= TOL_FP32_ABS, (what, stats)
    else:
        assert stats["max_rel_rms"] <= TOL_16BIT_REL_RMS, (what, stats)
    return stats


class Case:
    """One workload on both sides. `S` truncates workloads 2-4 for speed."""

    def __init__(self, cfg: int, S: Optional[int] = None, poison: bool = True,
                 partition_size: int = 0, seed: Optional[int] = None, block_size: int = 16):
        self.w = w = make_workload(cfg, seed=seed, S=S, block_size=block_size)
        self.sp = sp = w.spec
        self.dt = sp.dtype
        self.kdt = sp.cache_dtype        # the pools' storage type
        self.partition_size = partition_size
        log(f"[case] workload {cfg} {sp.name} S={sp.S} Hq={sp.Hq} Hkv={sp.Hkv} D={sp.D} "
            f"{sp.dtype} blocks={w.num_blocks} max_ctx={int(w.context_lens.max())}")
        values = self._values()
        # dry run of the oracle block manager to learn which slots end up
        # live and which get written, so the shared input pool can be poisoned
        B = self.B = sp.block_size
        dry = BlockManager(w.num_blocks, block_size=B, free_order=w.free_order)
        h = {}
        written = []
        for is_step, ops in ((False, w.setup_ops), (True, w.step_ops)):
            for op in ops:
                if op[0] == "create":
                    h[op[1]] = dry.create()
                elif op[0] == "fork":
                    h[op[2]] = dry.fork(h[op[1]])
                else:
                    slots, _ = dry.append(h[op[1]], op[2])
                    if is_step or (len(op) > 3 and op[3] == "values"):
                        written.extend(slots)
        live = np.zeros((w.num_blocks, B), bool)
        for s in range(sp.S):
            t = dry.table(h[s])
            for p in range(dry.length(h[s])):
                live[t[p // B], p % B] = True
        self.k_in, self.v_in = w.k_pool.copy(), w.v_pool.copy()
        if poison:
            dead = np.argwhere(~live)
            wr = np.array(written, dtype=np.int64)
            for pool in (self.k_in, self.v_in):
                if len(dead):
                    poison_slots(pool, self.kdt, dead[:, 0], dead[:, 1])
                if len(wr):
                    poison_slots(pool, self.kdt, wr // B, wr % B)
        self._oracle_side(values)

    def _values(self) -> Dict[int, Tuple[np.ndarray, np.ndarray]]:
        w = self.w
        if w.tail_k is None:
            return {}
        return {s: (w.tail_k[s], w.tail_v[s]) for s in range(self.sp.S)}

    def _oracle_side(self, values):
        w = self.w
        bm = BlockManager(w.num_blocks, block_size=self.B, free_order=w.free_order)
        kp, vp = self.k_in.copy(), self.v_in.copy()
        h = {}
        self.setup_pairs = []
        for op in w.setup_ops:
            if op[0] == "create":
                h[op[1]] = bm.create()
            elif op[0] == "fork":
                h[op[2]] = bm.fork(h[op[1]])
            else:
                slots, pairs = bm.append(h[op[1]], op[2])
                if pairs:
                    oa.copy_blocks([kp, vp], pairs)
                    self.setup_pairs.extend(pairs)
                if len(op) > 3 and op[3] == "values":
                    self._oracle_write(values[op[1]][0], values[op[1]][1], kp, vp, slots)
        step_slots = []
        for op in w.step_ops:
            slots, pairs = bm.append(h[op[1]], op[2])
            assert not pairs
            step_slots.extend(slots)
        self.step_slots = np.array(step_slots, dtype=np.int64)
        self._oracle_write(w.k_new, w.v_new, kp, vp, self.step_slots)
        self.tables, self.lens = bm.packed_tables([h[s] for s in range(self.sp.S)])
        self.k_ref, self.v_ref = kp, vp
        self.bm, self.oh = bm, h

    def _oracle_write(self, k, v, kp, vp, slots):
        if self.kdt == "e4m3":
            ofp8.reshape_and_cache_fp8(k, v, kp, vp, slots, self.dt, self.sp.k_scale,
                                       self.sp.v_scale, block_size=self.B)
        else:
            oa.reshape_and_cache(k, v, kp, vp, slots, block_size=self.B)

    def oracle_out(self, pairs: Optional[List[Tuple[int, int]]] = None) -> np.ndarray:
        if self.kdt == "e4m3":
            return oracle.decode_attention(self.w.q, self.k_ref, self.v_ref, self.tables,
                                           self.lens, self.sp.scale, self.dt, block_size=self.B,
                                           pairs=pairs, kv_dtype="e4m3",
                                           k_scale=self.sp.k_scale, v_scale=self.sp.v_scale)
        return oracle.decode_attention(self.w.q, self.k_ref, self.v_ref, self.tables, self.lens,
                                       self.sp.scale, self.dt, block_size=self.B, pairs=pairs)

    # -- device side ----------------------------------------------------------
    def device_run(self, partition_size: Optional[int] = None, fused: bool = True,
                   shared_prefix: bool = True):
        import torch
        from paged_kv_cache_162_amd.session import DecodeSession
        w, sp, dt = self.w, self.sp, self.dt
        self.k_dev = to_dev(self.k_in, self.kdt)
        self.v_dev = to_dev(self.v_in, self.kdt)
        ps = self.partition_size if partition_size is None else partition_size
        sess = DecodeSession(k_pool=self.k_dev, v_pool=self.v_dev, num_q_heads=sp.Hq,
                             free_order=w.free_order, partition_size=ps, fused=fused,
                             k_scale=sp.k_scale, v_scale=sp.v_scale, shared_prefix=shared_prefix)
        values = {}
        if w.tail_k is not None:
            values = {s: (to_dev(w.tail_k[s], dt), to_dev(w.tail_v[s], dt)) for s in range(sp.S)}
        cows = sess.run_ops(w.setup_ops, values)
        host_slots, step_pairs = sess.prepare_step(list(range(sp.S)))
        self.q_dev = to_dev(w.q, dt)
        self.kn_dev, self.vn_dev = to_dev(w.k_new, dt), to_dev(w.v_new, dt)
        self.out_dev = torch.full((sp.S, sp.Hq, sp.D), float("nan"), dtype=torch.float32,
                                  device="cuda")
        sess.step(self.q_dev, self.kn_dev, self.vn_dev, self.out_dev, sp.scale)
        torch.cuda.synchronize()
        self.sess = sess
        return cows, host_slots, step_pairs
