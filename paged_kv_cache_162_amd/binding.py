"""ctypes binding of libpagedkv.so: the C ABI's names, argument marshalling only.

Host functions take Python ints / sequences / numpy arrays. Device functions
take torch tensors that live on the GPU (PyTorch supplies device memory and
the stream); every computation happens inside the library's HIP kernels.
Errors raise KVError carrying the status name and kv_last_error()'s text.
There is no fallback: if the library is missing, importing this module fails.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

KV_OK, KV_ERR_INVALID, KV_ERR_OOM, KV_ERR_UNSUPPORTED, KV_ERR_HIP, KV_ERR_STATE = 0, -1, -2, -3, -4, -5
STATUS_NAMES = {0: "OK", -1: "INVALID", -2: "OOM", -3: "UNSUPPORTED", -4: "HIP", -5: "STATE"}
KV_F32, KV_F16, KV_BF16, KV_FP8_E4M3 = 0, 1, 2, 3
KV_LOADS_STREAM, KV_LOADS_CACHED = 0, 1
DTYPE_CODES = {"f32": KV_F32, "f16": KV_F16, "bf16": KV_BF16, "e4m3": KV_FP8_E4M3}
ELEM_BYTES = {KV_F32: 4, KV_F16: 2, KV_BF16: 2, KV_FP8_E4M3: 1}


class KVError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        self.status = status
        self.code = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{where}: {self.code}: {msg}")


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python paged_kv_cache_162_amd/build.py`")
    # torch first: its wheel carries its own HIP runtime under the same soname
    # (libamdhip64.so.7), and the library must bind to the runtime that owns
    # the tensors it is handed. Loaded the other way round, the first kernel
    # launch finds no device.
    import torch  # noqa: F401
    return C.CDLL(LIB_PATH)


lib = _load()

i32, i64, u64, f32, vp = C.c_int32, C.c_int64, C.c_uint64, C.c_float, C.c_void_p
P_i32, P_i64 = C.POINTER(C.c_int32), C.POINTER(C.c_int64)


class kv_pool_config(C.Structure):
    _fields_ = [("num_blocks", i32), ("block_size", i32), ("num_layers", i32),
                ("num_kv_heads", i32), ("head_dim", i32), ("dtype", C.c_int)]


_SIGS = {
    "kv_pool_create": (C.c_int, [C.POINTER(kv_pool_config), C.POINTER(vp)]),
    "kv_pool_destroy": (None, [vp]),
    "kv_pool_set_free_order": (C.c_int, [vp, i32, P_i32]),
    "kv_pool_layer_bytes": (C.c_size_t, [vp]),
    "kv_pool_capacity_tokens": (i64, [vp]),
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
    "kv_slot_mapping": (C.c_int, [vp, i32, i32, vp, vp, i32, i32, vp, vp]),
    "kv_reshape_and_cache": (C.c_int, [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, C.c_int, vp]),
    "kv_append_tokens": (C.c_int, [vp, i32, i32, vp, vp, i32, vp, vp, vp, vp, i32, i32, i32, i32,
                                   C.c_int, vp, vp]),
    "kv_copy_blocks": (C.c_int, [C.POINTER(vp), C.POINTER(vp), i32, vp, i32, i32, C.c_size_t, vp]),
    "kv_swap_out_blocks": (C.c_int, [C.POINTER(vp), C.POINTER(vp), i32, vp, i32, i32, C.c_size_t,
                                     vp, vp]),
    "kv_swap_in_blocks": (C.c_int, [C.POINTER(vp), C.POINTER(vp), i32, vp, i32, i32, C.c_size_t,
                                    vp, vp]),
    "kv_paged_attention_plan": (C.c_int, [P_i32, i32, i32, i32, i32, P_i32, i32, P_i32]),
    "kv_paged_attention_workspace_bytes": (C.c_size_t, [i32, i32, i32, i32, i32, i32]),
    "kv_paged_attention_decode": (C.c_int, [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32,
                                            i32, f32, C.c_int, i32, i32, vp, i32, vp, C.c_size_t,
                                            C.c_int, vp]),
    "kv_paged_attention_decode_append": (C.c_int, [vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32,
                                                   i32, i32, i32, i32, f32, C.c_int, i32, i32,
                                                   vp, i32, vp, C.c_size_t, vp, C.c_int, vp]),
    "kv_paged_attention_decode_append_noalloc": (C.c_int, [vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                                           i32, i32, i32, i32, i32, i32, f32,
                                                           C.c_int, i32, i32, vp, i32, vp,
                                                           C.c_int, vp]),
    "kv_paged_attention_shared_aux_bytes": (C.c_size_t, [i32, i32, i32, i32, i32]),
    "kv_paged_attention_decode_append_shared": (C.c_int, [vp, vp, vp, vp, vp, vp, vp, i32, vp, i32,
                                                          i32, i32, i32, i32, i32, f32, C.c_int,
                                                          i32, i32, i32, vp, i32, vp, C.c_size_t,
                                                          vp, C.c_size_t, vp, C.c_int, vp]),
    "kv_reshape_and_cache_fp8": (C.c_int, [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, C.c_int,
                                           f32, f32, vp]),
    "kv_quantize_fp8": (C.c_int, [vp, vp, i64, C.c_int, f32, vp]),
    "kv_paged_attention_decode_fp8": (C.c_int, [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32,
                                                i32, i32, f32, C.c_int, f32, f32, i32, i32, vp,
                                                i32, vp, C.c_size_t, C.c_int, vp]),
    "kv_paged_attention_decode_append_fp8": (C.c_int, [vp, vp, vp, vp, vp, vp, vp, i32, vp, i32,
                                                       i32, i32, i32, i32, i32, f32, C.c_int, f32,
                                                       f32, i32, i32, vp, i32, vp, C.c_size_t, vp,
                                                       C.c_int, vp]),
    "kv_paged_attention_decode_append_shared_fp8": (C.c_int, [vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                                              i32, i32, i32, i32, i32, i32, f32,
                                                              C.c_int, f32, f32, i32, i32, i32, vp,
                                                              i32, vp, C.c_size_t, vp, C.c_size_t,
                                                              vp, C.c_int, vp]),
    "kv_paged_attention_prefill_rows_per_item": (i32, [i32, i32]),
    "kv_paged_attention_prefill_plan": (C.c_int, [P_i32, P_i32, i32, i32, i32, P_i32, i32, P_i32]),
    "kv_paged_attention_prefill": (C.c_int, [vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32,
                                             i32, i32, i32, f32, C.c_int, i32, vp, i32, vp]),
    "kv_paged_attention_prefill_fp8": (C.c_int, [vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32,
                                                 i32, i32, i32, i32, f32, C.c_int, f32, f32, i32,
                                                 vp, i32, vp]),
    "kv_paged_attention_prefill_choose_splits": (i32, [P_i32, P_i32, i32, i32, i32, i32]),
    "kv_paged_attention_prefill_workspace_bytes": (C.c_size_t, [i32, i32, i32, i32]),
    "kv_paged_attention_prefill_split": (C.c_int, [vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32,
                                                   i32, i32, i32, i32, f32, C.c_int, i32, vp, i32,
                                                   i32, vp, C.c_size_t, vp]),
    "kv_paged_attention_prefill_split_fp8": (C.c_int, [vp, vp, vp, vp, vp, i32, vp, vp, i32, i32,
                                                       i32, i32, i32, i32, i32, f32, C.c_int, f32,
                                                       f32, i32, vp, i32, i32, vp, C.c_size_t,
                                                       vp]),
    "kv_paged_attention_choose_partition": (i32, [P_i32, i32, i32, i32, i32]),
    "kv_paged_attention_common_prefix": (i32, [P_i32, i32, i32, P_i32, i32]),
    "kv_paged_attention_choose_shared_prefix": (i32, [P_i32, i32, i32, P_i32, i32, i32, i32, i32,
                                                      C.c_int]),
    "kv_paged_attention_choose_load_policy": (C.c_int, [vp, i32]),
    "kv_hbm_read_probe": (C.c_int, [vp, C.c_size_t, vp, i32, vp]),
    "kv_last_error": (C.c_char_p, []),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


def _check(status: int, where: str) -> None:
    if status != KV_OK:
        raise KVError(status, where, lib.kv_last_error().decode())


def _i32_array(xs) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(xs, dtype=np.int32))


def _p32(a: np.ndarray):
    return a.ctypes.data_as(P_i32)


# ---------------------------------------------------------------------------
# host: pool and blocks
# ---------------------------------------------------------------------------
def kv_pool_create(num_blocks: int, block_size: int = 16, num_layers: int = 1,
                   num_kv_heads: int = 1, head_dim: int = 128, dtype: int = KV_BF16) -> int:
    cfg = kv_pool_config(num_blocks, block_size, num_layers, num_kv_heads, head_dim, dtype)
    h = vp()
    _check(lib.kv_pool_create(C.byref(cfg), C.byref(h)), "kv_pool_create")
    return h.value


def kv_pool_destroy(pool: int) -> None:
    lib.kv_pool_destroy(pool)


def kv_pool_set_free_order(pool: int, order: Sequence[int]) -> None:
    a = _i32_array(order)
    _check(lib.kv_pool_set_free_order(pool, len(a), _p32(a)), "kv_pool_set_free_order")


def kv_pool_layer_bytes(pool: int) -> int:
    return int(lib.kv_pool_layer_bytes(pool))


def kv_pool_capacity_tokens(pool: int) -> int:
    return int(lib.kv_pool_capacity_tokens(pool))


def kv_num_free_blocks(pool: int) -> int:
    return int(lib.kv_num_free_blocks(pool))


def kv_block_alloc(pool: int, n: int) -> np.ndarray:
    out = np.zeros(max(n, 0), dtype=np.int32)
    _check(lib.kv_block_alloc(pool, n, _p32(out)), "kv_block_alloc")
    return out


def kv_block_incref(pool: int, ids: Sequence[int]) -> None:
    a = _i32_array(ids)
    _check(lib.kv_block_incref(pool, len(a), _p32(a)), "kv_block_incref")


def kv_block_free(pool: int, ids: Sequence[int]) -> None:
    a = _i32_array(ids)
    _check(lib.kv_block_free(pool, len(a), _p32(a)), "kv_block_free")


def kv_block_refcount(pool: int, block: int) -> int:
    return int(lib.kv_block_refcount(pool, block))


# ---------------------------------------------------------------------------
# host: sequences
# ---------------------------------------------------------------------------
def kv_seq_create(pool: int) -> int:
    s = i64()
    _check(lib.kv_seq_create(pool, C.byref(s)), "kv_seq_create")
    return s.value


def kv_seq_fork(pool: int, parent: int) -> int:
    s = i64()
    _check(lib.kv_seq_fork(pool, parent, C.byref(s)), "kv_seq_fork")
    return s.value


def kv_seq_append(pool: int, seq: int, n_tokens: int) -> Tuple[np.ndarray, Optional[Tuple[int, int]]]:
    """Returns (slots int64 [n_tokens], (src, dst) copy-on-write pair or None)."""
    slots = np.zeros(max(n_tokens, 1), dtype=np.int64)
    src, dst, n = i32(), i32(), i32()
    _check(lib.kv_seq_append(pool, seq, n_tokens, slots.ctypes.data_as(P_i64),
                             C.byref(src), C.byref(dst), C.byref(n)), "kv_seq_append")
    return slots[:max(n_tokens, 0)], ((src.value, dst.value) if n.value else None)


def kv_seq_free(pool: int, seq: int) -> None:
    _check(lib.kv_seq_free(pool, seq), "kv_seq_free")


def kv_seq_block_table(pool: int, seq: int) -> np.ndarray:
    n = i32()
    st = lib.kv_seq_block_table(pool, seq, 0, None, C.byref(n))
    if st == KV_ERR_STATE:
        _check(st, "kv_seq_block_table")
    out = np.zeros(max(n.value, 1), dtype=np.int32)
    _check(lib.kv_seq_block_table(pool, seq, len(out), _p32(out), C.byref(n)), "kv_seq_block_table")
    return out[:n.value]


def kv_seq_len(pool: int, seq: int) -> int:
    return int(lib.kv_seq_len(pool, seq))


def kv_seq_pack_tables(pool: int, seqs: Sequence[int], max_blocks: int) -> Tuple[np.ndarray, np.ndarray]:
    s = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
    tables = np.zeros((len(s), max_blocks), dtype=np.int32)
    lens = np.zeros(len(s), dtype=np.int32)
    _check(lib.kv_seq_pack_tables(pool, len(s), s.ctypes.data_as(P_i64), max_blocks,
                                  _p32(tables), _p32(lens)), "kv_seq_pack_tables")
    return tables, lens


def _seq_ids(fn, where: str, pool: int, seq: int) -> np.ndarray:
    """Call a (pool, seq, cap, ids, n) entry point, sizing ids from *n."""
    n = i32()
    cap = max(kv_seq_len(pool, seq), 0) + 1  # ceil(len / B) <= len + 1 blocks
    out = np.zeros(cap, dtype=np.int32)
    _check(fn(pool, seq, cap, _p32(out), C.byref(n)), where)
    return out[:n.value]


def kv_seq_swap_out(pool: int, seq: int) -> np.ndarray:
    """Release `seq`'s blocks for a swap; returns the table to copy out."""
    return _seq_ids(lib.kv_seq_swap_out, "kv_seq_swap_out", pool, seq)


def kv_seq_swap_in(pool: int, seq: int) -> np.ndarray:
    """Give a swapped-out `seq` fresh blocks; returns them in logical order."""
    return _seq_ids(lib.kv_seq_swap_in, "kv_seq_swap_in", pool, seq)


def kv_seq_is_swapped(pool: int, seq: int) -> int:
    return int(lib.kv_seq_is_swapped(pool, seq))


def kv_pool_shared_blocks(pool: int) -> int:
    return int(lib.kv_pool_shared_blocks(pool))


def kv_paged_attention_choose_partition(context_lens_host, num_kv_heads: int, block_size: int,
                                        min_units: int) -> int:
    lens = _i32_array(context_lens_host)
    return int(lib.kv_paged_attention_choose_partition(_p32(lens), len(lens), num_kv_heads,
                                                        block_size, min_units))


def kv_paged_attention_common_prefix(tables_host, context_lens_host, block_size: int) -> int:
    """Positions every sequence reaches through the same leading blocks (whole blocks,
    short of each sequence's last position)."""
    tab = np.ascontiguousarray(tables_host, dtype=np.int32)
    lens = _i32_array(context_lens_host)
    return int(lib.kv_paged_attention_common_prefix(_p32(tab), tab.shape[0], tab.shape[1],
                                                    _p32(lens), block_size))


def kv_paged_attention_choose_shared_prefix(tables_host, context_lens_host, block_size: int,
                                            num_q_heads: int, num_kv_heads: int, head_dim: int,
                                            dtype: int) -> int:
    """Shared positions for the shared-prefix step, or 0 for the plain step."""
    tab = np.ascontiguousarray(tables_host, dtype=np.int32)
    lens = _i32_array(context_lens_host)
    return int(lib.kv_paged_attention_choose_shared_prefix(
        _p32(tab), tab.shape[0], tab.shape[1], _p32(lens), block_size, num_q_heads, num_kv_heads,
        head_dim, dtype))


def kv_paged_attention_choose_load_policy(pool: int, shared_tokens: int) -> int:
    return int(lib.kv_paged_attention_choose_load_policy(pool, shared_tokens))


# ---------------------------------------------------------------------------
# device entry points (torch tensors on the GPU)
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    return {torch.float32: KV_F32, torch.float16: KV_F16, torch.bfloat16: KV_BF16,
            torch.uint8: KV_FP8_E4M3}[t.dtype]


def _dev(t, name: str, dtype=None):
    if not t.is_cuda:
        raise KVError(KV_ERR_INVALID, name, "tensor must live on the GPU")
    if not t.is_contiguous():
        raise KVError(KV_ERR_INVALID, name, "tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise KVError(KV_ERR_INVALID, name, f"expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def kv_slot_mapping(tables, seq_idx, pos, slots, block_size: int = 16, stream=None) -> None:
    torch = _torch()
    _check(lib.kv_slot_mapping(_dev(tables, "tables", torch.int32), tables.shape[0], tables.shape[1],
                               _dev(seq_idx, "seq_idx", torch.int32), _dev(pos, "pos", torch.int32),
                               pos.numel(), block_size, _dev(slots, "slots", torch.int64),
                               _stream(stream)), "kv_slot_mapping")


def kv_reshape_and_cache(k_new, v_new, k_pool, v_pool, slots, stream=None) -> None:
    """k_new/v_new [n, Hkv, D]; k_pool/v_pool [NB, Hkv, B, D]; slots int64 [n]."""
    torch = _torch()
    NB, Hkv, B, D = k_pool.shape
    if tuple(v_pool.shape) != tuple(k_pool.shape) or k_new.shape != v_new.shape \
            or k_new.shape[1:] != (Hkv, D) or k_new.dtype != k_pool.dtype:
        raise KVError(KV_ERR_INVALID, "kv_reshape_and_cache", "shape/dtype mismatch")
    _check(lib.kv_reshape_and_cache(_dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(k_pool, "k_pool"),
                                    _dev(v_pool, "v_pool"), _dev(slots, "slots", torch.int64),
                                    k_new.shape[0], NB, Hkv, D, B, dtype_code(k_pool), _stream(stream)),
           "kv_reshape_and_cache")


def kv_append_tokens(tables, seq_idx, pos, k_new, v_new, k_pool, v_pool, slots, stream=None) -> None:
    """Slot mapping + cache write in one launch. tables int32 [rows, max_blocks];
    seq_idx/pos int32 [n]; k_new/v_new [n, Hkv, D]; pools [NB, Hkv, B, D];
    slots int64 [n] (output)."""
    torch = _torch()
    NB, Hkv, B, D = k_pool.shape
    if tuple(v_pool.shape) != tuple(k_pool.shape) or k_new.shape != v_new.shape \
            or k_new.shape[1:] != (Hkv, D) or k_new.dtype != k_pool.dtype \
            or seq_idx.numel() != k_new.shape[0] or pos.numel() != k_new.shape[0] \
            or slots.numel() != k_new.shape[0]:
        raise KVError(KV_ERR_INVALID, "kv_append_tokens", "shape/dtype mismatch")
    _check(lib.kv_append_tokens(_dev(tables, "tables", torch.int32), tables.shape[0], tables.shape[1],
                                _dev(seq_idx, "seq_idx", torch.int32), _dev(pos, "pos", torch.int32),
                                k_new.shape[0], _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                                _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), NB, Hkv, D, B,
                                dtype_code(k_pool), _dev(slots, "slots", torch.int64), _stream(stream)),
           "kv_append_tokens")


def kv_copy_blocks(k_pools: List, v_pools: List, pairs, num_blocks: int, block_bytes: int,
                   stream=None) -> None:
    """pairs: device int32 tensor [n, 2] of (src, dst) block IDs."""
    torch = _torch()
    L = len(k_pools)
    if len(v_pools) != L:
        raise KVError(KV_ERR_INVALID, "kv_copy_blocks", "k_pools and v_pools differ in length")
    kp = (vp * max(L, 1))(*[_dev(t, "k_pools") for t in k_pools])
    vv = (vp * max(L, 1))(*[_dev(t, "v_pools") for t in v_pools])
    _check(lib.kv_copy_blocks(kp, vv, L, _dev(pairs, "pairs", torch.int32), pairs.shape[0],
                              num_blocks, block_bytes, _stream(stream)), "kv_copy_blocks")


def _swap(fn, where: str, k_pools: List, v_pools: List, block_ids, num_blocks: int,
          block_bytes: int, host, stream) -> None:
    torch = _torch()
    L = len(k_pools)
    if len(v_pools) != L:
        raise KVError(KV_ERR_INVALID, where, "k_pools and v_pools differ in length")
    if host.is_cuda or not host.is_contiguous():
        raise KVError(KV_ERR_INVALID, where, "host buffer must be a contiguous CPU tensor")
    kp = (vp * max(L, 1))(*[_dev(t, "k_pools") for t in k_pools])
    vv = (vp * max(L, 1))(*[_dev(t, "v_pools") for t in v_pools])
    n = block_ids.shape[0]
    if host.numel() * host.element_size() < n * L * 2 * block_bytes:
        raise KVError(KV_ERR_INVALID, where, "host buffer too small")
    _check(fn(kp, vv, L, _dev(block_ids, "block_ids", torch.int32), n, num_blocks, block_bytes,
              host.data_ptr(), _stream(stream)), where)


def kv_swap_out_blocks(k_pools: List, v_pools: List, block_ids, num_blocks: int,
                       block_bytes: int, host, stream=None) -> None:
    """Copy blocks (all layers, K and V) into pinned `host`
    [n][layers][2][block_bytes]; block_ids: device int32 tensor [n]."""
    _swap(lib.kv_swap_out_blocks, "kv_swap_out_blocks", k_pools, v_pools, block_ids,
          num_blocks, block_bytes, host, stream)


def kv_swap_in_blocks(k_pools: List, v_pools: List, block_ids, num_blocks: int,
                      block_bytes: int, host, stream=None) -> None:
    """Copy pinned `host` [n][layers][2][block_bytes] back into blocks."""
    _swap(lib.kv_swap_in_blocks, "kv_swap_in_blocks", k_pools, v_pools, block_ids,
          num_blocks, block_bytes, host, stream)


def kv_hbm_read_probe(src, sink, workgroups: int, stream=None) -> None:
    """Stream-read every byte of device tensor src; sink: device uint32/int32 [workgroups]."""
    _check(lib.kv_hbm_read_probe(_dev(src, "src"), src.numel() * src.element_size(),
                                 _dev(sink, "sink"), workgroups, _stream(stream)),
           "kv_hbm_read_probe")


def kv_paged_attention_plan(context_lens_host, partition_size: int = 0, num_kv_heads: int = 0,
                            num_cus: int = 0) -> np.ndarray:
    """Host work plan: int32 [n_items, 2] (sequence, partition), longest first,
    laid out for the workgroup placement of a device with num_cus compute units
    (0 = plain longest-first order)."""
    lens = _i32_array(context_lens_host)
    n = i32()
    st = lib.kv_paged_attention_plan(_p32(lens), len(lens), partition_size, num_kv_heads,
                                     num_cus, None, 0, C.byref(n))
    if st != KV_OK and n.value == 0:
        _check(st, "kv_paged_attention_plan")
    out = np.zeros((max(n.value, 1), 2), dtype=np.int32)
    _check(lib.kv_paged_attention_plan(_p32(lens), len(lens), partition_size, num_kv_heads,
                                       num_cus, _p32(out), out.shape[0], C.byref(n)),
           "kv_paged_attention_plan")
    return out[:n.value]


def kv_paged_attention_workspace_bytes(S: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                                       max_context_len: int, partition_size: int = 0) -> int:
    return int(lib.kv_paged_attention_workspace_bytes(S, num_q_heads, num_kv_heads, head_dim,
                                                       max_context_len, partition_size))


def kv_paged_attention_decode(out, q, k_pool, v_pool, block_tables, context_lens, scale: float,
                              max_context_len: int, workspace=None, partition_size: int = 0,
                              work_items=None, load_policy: int = KV_LOADS_STREAM,
                              stream=None) -> None:
    """out fp32 [S, Hq, D]; q [S, Hq, D]; pools [NB, Hkv, B, D]; tables int32 [S, max_blocks];
    context_lens int32 [S]; workspace: uint8/any device tensor or None; work_items: device
    int32 [n, 2] from kv_paged_attention_plan or None."""
    torch = _torch()
    S, Hq, D = q.shape
    NB, Hkv, B, D2 = k_pool.shape
    if D2 != D or tuple(out.shape) != (S, Hq, D) or block_tables.shape[0] != S \
            or context_lens.numel() != S or q.dtype != k_pool.dtype or v_pool.shape != k_pool.shape:
        raise KVError(KV_ERR_INVALID, "kv_paged_attention_decode", "shape/dtype mismatch")
    ws_ptr, ws_bytes = (0, 0) if workspace is None else (_dev(workspace, "workspace"),
                                                         workspace.numel() * workspace.element_size())
    _check(lib.kv_paged_attention_decode(
        _dev(out, "out", torch.float32), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), S, Hq, Hkv, D, B, NB, float(scale),
        dtype_code(q), partition_size, max_context_len,
        None if work_items is None else _dev(work_items, "work_items", torch.int32),
        0 if work_items is None else work_items.shape[0], ws_ptr or None, ws_bytes,
        int(load_policy), _stream(stream)),
        "kv_paged_attention_decode")


def kv_paged_attention_decode_append(out, q, k_new, v_new, k_pool, v_pool, block_tables,
                                     context_lens, scale: float, max_context_len: int, slots,
                                     workspace=None, partition_size: int = 0, work_items=None,
                                     load_policy: int = KV_LOADS_STREAM, stream=None) -> None:
    """Decode step with the cache write fused in: k_new/v_new [S, Hkv, D] are written at
    position context_lens[s]-1 of each sequence (slots int64 [S] receives the slots), then
    attention as kv_paged_attention_decode."""
    torch = _torch()
    S, Hq, D = q.shape
    NB, Hkv, B, D2 = k_pool.shape
    if D2 != D or tuple(out.shape) != (S, Hq, D) or block_tables.shape[0] != S \
            or context_lens.numel() != S or q.dtype != k_pool.dtype or v_pool.shape != k_pool.shape \
            or tuple(k_new.shape) != (S, Hkv, D) or k_new.shape != v_new.shape \
            or k_new.dtype != k_pool.dtype or slots.numel() != S:
        raise KVError(KV_ERR_INVALID, "kv_paged_attention_decode_append", "shape/dtype mismatch")
    ws_ptr, ws_bytes = (0, 0) if workspace is None else (_dev(workspace, "workspace"),
                                                         workspace.numel() * workspace.element_size())
    _check(lib.kv_paged_attention_decode_append(
        _dev(out, "out", torch.float32), _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), S, Hq, Hkv, D, B, NB, float(scale),
        dtype_code(q), partition_size, max_context_len,
        None if work_items is None else _dev(work_items, "work_items", torch.int32),
        0 if work_items is None else work_items.shape[0], ws_ptr or None, ws_bytes,
        _dev(slots, "slots", torch.int64), int(load_policy), _stream(stream)),
        "kv_paged_attention_decode_append")


KV_NOALLOC_SCRATCH_BYTES = 32 << 20


def kv_paged_attention_decode_append_noalloc(out, q, k_new, v_new, k_pool, v_pool, block_tables,
                                             context_lens, scale: float, max_context_len: int,
                                             slots, partition_size: int = 0, work_items=None,
                                             load_policy: int = KV_LOADS_STREAM,
                                             stream=None) -> None:
    """kv_paged_attention_decode_append with the split-K partials in the library's own
    per-GPU buffer (KV_NOALLOC_SCRATCH_BYTES) instead of a caller workspace."""
    torch = _torch()
    S, Hq, D = q.shape
    NB, Hkv, B, D2 = k_pool.shape
    if D2 != D or tuple(out.shape) != (S, Hq, D) or block_tables.shape[0] != S \
            or context_lens.numel() != S or q.dtype != k_pool.dtype or v_pool.shape != k_pool.shape \
            or tuple(k_new.shape) != (S, Hkv, D) or k_new.shape != v_new.shape \
            or k_new.dtype != k_pool.dtype or slots.numel() != S:
        raise KVError(KV_ERR_INVALID, "kv_paged_attention_decode_append_noalloc",
                      "shape/dtype mismatch")
    _check(lib.kv_paged_attention_decode_append_noalloc(
        _dev(out, "out", torch.float32), _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), S, Hq, Hkv, D, B, NB, float(scale),
        dtype_code(q), partition_size, max_context_len,
        None if work_items is None else _dev(work_items, "work_items", torch.int32),
        0 if work_items is None else work_items.shape[0], _dev(slots, "slots", torch.int64),
        int(load_policy), _stream(stream)),
        "kv_paged_attention_decode_append_noalloc")


KV_SHARED_PREFIX_MAX_TOKENS = 131072


def kv_paged_attention_shared_aux_bytes(S: int, num_q_heads: int, num_kv_heads: int,
                                        head_dim: int, shared_tokens: int) -> int:
    return int(lib.kv_paged_attention_shared_aux_bytes(S, num_q_heads, num_kv_heads, head_dim,
                                                       shared_tokens))


def kv_paged_attention_decode_append_shared(out, q, k_new, v_new, k_pool, v_pool, block_tables,
                                            context_lens, scale: float, shared_tokens: int,
                                            max_tail_len: int, slots, aux, workspace=None,
                                            partition_size: int = 0, work_items=None,
                                            load_policy: int = KV_LOADS_STREAM,
                                            stream=None) -> None:
    """kv_paged_attention_decode_append for sequences sharing their first shared_tokens
    positions: attention over the shared positions computed once for all queries, the tails
    per sequence; aux: device tensor of kv_paged_attention_shared_aux_bytes bytes; work_items
    and workspace are for the tails (lengths context_lens - shared_tokens)."""
    torch = _torch()
    S, Hq, D = q.shape
    NB, Hkv, B, D2 = k_pool.shape
    if D2 != D or tuple(out.shape) != (S, Hq, D) or block_tables.shape[0] != S \
            or context_lens.numel() != S or q.dtype != k_pool.dtype or v_pool.shape != k_pool.shape \
            or tuple(k_new.shape) != (S, Hkv, D) or k_new.shape != v_new.shape \
            or k_new.dtype != k_pool.dtype or slots.numel() != S:
        raise KVError(KV_ERR_INVALID, "kv_paged_attention_decode_append_shared",
                      "shape/dtype mismatch")
    ws_ptr, ws_bytes = (0, 0) if workspace is None else (_dev(workspace, "workspace"),
                                                         workspace.numel() * workspace.element_size())
    _check(lib.kv_paged_attention_decode_append_shared(
        _dev(out, "out", torch.float32), _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), S, Hq, Hkv, D, B, NB, float(scale),
        dtype_code(q), partition_size, shared_tokens, max_tail_len,
        None if work_items is None else _dev(work_items, "work_items", torch.int32),
        0 if work_items is None else work_items.shape[0], ws_ptr or None, ws_bytes,
        _dev(aux, "aux"), aux.numel() * aux.element_size(), _dev(slots, "slots", torch.int64),
        int(load_policy), _stream(stream)),
        "kv_paged_attention_decode_append_shared")


# ---------------------------------------------------------------------------
# fp8 (E4M3) cache: pools are uint8 tensors of codes, one scale per pool
# ---------------------------------------------------------------------------
def _fp8_pools(where, k_pool, v_pool):
    torch = _torch()
    if k_pool.dtype != torch.uint8 or v_pool.dtype != torch.uint8 or v_pool.shape != k_pool.shape:
        raise KVError(KV_ERR_INVALID, where, "fp8 pools must be matching uint8 tensors")
    return k_pool.shape


def kv_reshape_and_cache_fp8(k_new, v_new, k_pool, v_pool, slots, k_scale: float,
                             v_scale: float, stream=None) -> None:
    """k_new/v_new f16/bf16 [n, Hkv, D] -> uint8 pools [NB, Hkv, B, D], quantised."""
    torch = _torch()
    NB, Hkv, B, D = _fp8_pools("kv_reshape_and_cache_fp8", k_pool, v_pool)
    if k_new.shape != v_new.shape or k_new.shape[1:] != (Hkv, D) or k_new.dtype != v_new.dtype:
        raise KVError(KV_ERR_INVALID, "kv_reshape_and_cache_fp8", "shape/dtype mismatch")
    _check(lib.kv_reshape_and_cache_fp8(
        _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(slots, "slots", torch.int64), k_new.shape[0], NB, Hkv, D, B, dtype_code(k_new),
        float(k_scale), float(v_scale), _stream(stream)), "kv_reshape_and_cache_fp8")


def kv_quantize_fp8(src, dst, scale: float, stream=None) -> None:
    """dst uint8 (same number of elements) = E4M3 codes of src (f16/bf16) / scale."""
    torch = _torch()
    if dst.dtype != torch.uint8 or dst.numel() != src.numel():
        raise KVError(KV_ERR_INVALID, "kv_quantize_fp8", "dst must be uint8 with src's size")
    _check(lib.kv_quantize_fp8(_dev(src, "src"), _dev(dst, "dst"), src.numel(), dtype_code(src),
                               float(scale), _stream(stream)), "kv_quantize_fp8")


def kv_paged_attention_decode_fp8(out, q, k_pool, v_pool, block_tables, context_lens,
                                  scale: float, k_scale: float, v_scale: float,
                                  max_context_len: int, workspace=None, partition_size: int = 0,
                                  work_items=None, load_policy: int = KV_LOADS_STREAM,
                                  stream=None) -> None:
    """kv_paged_attention_decode over uint8 E4M3 pools with per-pool scales; q f16/bf16."""
    torch = _torch()
    S, Hq, D = q.shape
    NB, Hkv, B, D2 = _fp8_pools("kv_paged_attention_decode_fp8", k_pool, v_pool)
    if D2 != D or tuple(out.shape) != (S, Hq, D) or block_tables.shape[0] != S \
            or context_lens.numel() != S:
        raise KVError(KV_ERR_INVALID, "kv_paged_attention_decode_fp8", "shape mismatch")
    ws_ptr, ws_bytes = (0, 0) if workspace is None else (_dev(workspace, "workspace"),
                                                         workspace.numel() * workspace.element_size())
    _check(lib.kv_paged_attention_decode_fp8(
        _dev(out, "out", torch.float32), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), S, Hq, Hkv, D, B, NB, float(scale),
        dtype_code(q), float(k_scale), float(v_scale), partition_size, max_context_len,
        None if work_items is None else _dev(work_items, "work_items", torch.int32),
        0 if work_items is None else work_items.shape[0], ws_ptr or None, ws_bytes,
        int(load_policy), _stream(stream)),
        "kv_paged_attention_decode_fp8")


def kv_paged_attention_decode_append_fp8(out, q, k_new, v_new, k_pool, v_pool, block_tables,
                                         context_lens, scale: float, k_scale: float,
                                         v_scale: float, max_context_len: int, slots,
                                         workspace=None, partition_size: int = 0,
                                         work_items=None, load_policy: int = KV_LOADS_STREAM,
                                         stream=None) -> None:
    """Fused decode step over uint8 E4M3 pools: the new token is quantised and written at
    position context_lens[s]-1, then attention as kv_paged_attention_decode_fp8."""
    torch = _torch()
    S, Hq, D = q.shape
    NB, Hkv, B, D2 = _fp8_pools("kv_paged_attention_decode_append_fp8", k_pool, v_pool)
    if D2 != D or tuple(out.shape) != (S, Hq, D) or block_tables.shape[0] != S \
            or context_lens.numel() != S or tuple(k_new.shape) != (S, Hkv, D) \
            or k_new.shape != v_new.shape or k_new.dtype != q.dtype or v_new.dtype != q.dtype \
            or slots.numel() != S:
        raise KVError(KV_ERR_INVALID, "kv_paged_attention_decode_append_fp8", "shape/dtype mismatch")
    ws_ptr, ws_bytes = (0, 0) if workspace is None else (_dev(workspace, "workspace"),
                                                         workspace.numel() * workspace.element_size())
    _check(lib.kv_paged_attention_decode_append_fp8(
        _dev(out, "out", torch.float32), _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), S, Hq, Hkv, D, B, NB, float(scale),
        dtype_code(q), float(k_scale), float(v_scale), partition_size, max_context_len,
        None if work_items is None else _dev(work_items, "work_items", torch.int32),
        0 if work_items is None else work_items.shape[0], ws_ptr or None, ws_bytes,
        _dev(slots, "slots", torch.int64), int(load_policy), _stream(stream)),
        "kv_paged_attention_decode_append_fp8")


def kv_paged_attention_decode_append_shared_fp8(out, q, k_new, v_new, k_pool, v_pool,
                                                block_tables, context_lens, scale: float,
                                                k_scale: float, v_scale: float,
                                                shared_tokens: int, max_tail_len: int, slots, aux,
                                                workspace=None, partition_size: int = 0,
                                                work_items=None,
                                                load_policy: int = KV_LOADS_STREAM,
                                                stream=None) -> None:
    """kv_paged_attention_decode_append_shared over uint8 E4M3 pools with per-pool scales;
    q, k_new, v_new f16/bf16."""
    torch = _torch()
    S, Hq, D = q.shape
    NB, Hkv, B, D2 = _fp8_pools("kv_paged_attention_decode_append_shared_fp8", k_pool, v_pool)
    if D2 != D or tuple(out.shape) != (S, Hq, D) or block_tables.shape[0] != S \
            or context_lens.numel() != S or tuple(k_new.shape) != (S, Hkv, D) \
            or k_new.shape != v_new.shape or k_new.dtype != q.dtype or v_new.dtype != q.dtype \
            or slots.numel() != S:
        raise KVError(KV_ERR_INVALID, "kv_paged_attention_decode_append_shared_fp8",
                      "shape/dtype mismatch")
    ws_ptr, ws_bytes = (0, 0) if workspace is None else (_dev(workspace, "workspace"),
                                                         workspace.numel() * workspace.element_size())
    _check(lib.kv_paged_attention_decode_append_shared_fp8(
        _dev(out, "out", torch.float32), _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), S, Hq, Hkv, D, B, NB, float(scale),
        dtype_code(q), float(k_scale), float(v_scale), partition_size, shared_tokens,
        max_tail_len, None if work_items is None else _dev(work_items, "work_items", torch.int32),
        0 if work_items is None else work_items.shape[0], ws_ptr or None, ws_bytes,
        _dev(aux, "aux"), aux.numel() * aux.element_size(), _dev(slots, "slots", torch.int64),
        int(load_policy), _stream(stream)),
        "kv_paged_attention_decode_append_shared_fp8")


# ---------------------------------------------------------------------------
# chunked prefill: several query tokens per sequence, causal within the chunk
# ---------------------------------------------------------------------------
def kv_paged_attention_prefill_rows_per_item(num_q_heads: int, num_kv_heads: int) -> int:
    return int(lib.kv_paged_attention_prefill_rows_per_item(num_q_heads, num_kv_heads))


def kv_paged_attention_prefill_plan(query_start_host, context_lens_host, num_q_heads: int,
                                    num_kv_heads: int) -> np.ndarray:
    """Host work plan: int32 [n_items, 2] (sequence, row block), most keys first."""
    qs = _i32_array(query_start_host)
    lens = _i32_array(context_lens_host)
    if len(qs) != len(lens) + 1:
        raise KVError(KV_ERR_INVALID, "kv_paged_attention_prefill_plan", "query_start needs S + 1 entries")
    n = i32()
    st = lib.kv_paged_attention_prefill_plan(_p32(qs), _p32(lens), len(lens), num_q_heads,
                                             num_kv_heads, None, 0, C.byref(n))
    if st != KV_OK and n.value == 0:
        _check(st, "kv_paged_attention_prefill_plan")
    out = np.zeros((max(n.value, 1), 2), dtype=np.int32)
    _check(lib.kv_paged_attention_prefill_plan(_p32(qs), _p32(lens), len(lens), num_q_heads,
                                               num_kv_heads, _p32(out), out.shape[0], C.byref(n)),
           "kv_paged_attention_prefill_plan")
    return out[:n.value]


def kv_paged_attention_prefill(out, q, k_pool, v_pool, block_tables, context_lens, query_start,
                               scale: float, max_query_len: int, work_items=None,
                               stream=None) -> None:
    """out fp32 [T, Hq, D]; q [T, Hq, D] f16/bf16; pools [NB, Hkv, B, D] of q's dtype;
    tables int32 [S, max_blocks]; context_lens int32 [S]; query_start int32 [S + 1]."""
    torch = _torch()
    T, Hq, D = q.shape
    NB, Hkv, B, D2 = k_pool.shape
    S = context_lens.numel()
    if D2 != D or tuple(out.shape) != (T, Hq, D) or block_tables.shape[0] != S \
            or query_start.numel() != S + 1 or q.dtype != k_pool.dtype \
            or v_pool.shape != k_pool.shape:
        raise KVError(KV_ERR_INVALID, "kv_paged_attention_prefill", "shape/dtype mismatch")
    _check(lib.kv_paged_attention_prefill(
        _dev(out, "out", torch.float32), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), _dev(query_start, "query_start", torch.int32),
        S, T, Hq, Hkv, D, B, NB, float(scale), dtype_code(q), max_query_len,
        None if work_items is None else _dev(work_items, "work_items", torch.int32),
        0 if work_items is None else work_items.shape[0], _stream(stream)),
        "kv_paged_attention_prefill")


KV_PREFILL_MAX_SPLITS = 64


def kv_paged_attention_prefill_choose_splits(query_start_host, context_lens_host, num_q_heads: int,
                                             num_kv_heads: int, min_units: int) -> int:
    """Key runs per block for a prefill launch (1 = no split)."""
    qs = _i32_array(query_start_host)
    lens = _i32_array(context_lens_host)
    if qs.size != lens.size + 1:
        raise KVError(KV_ERR_INVALID, "kv_paged_attention_prefill_choose_splits",
                      "query_start needs S + 1 entries")
    return int(lib.kv_paged_attention_prefill_choose_splits(_p32(qs), _p32(lens), len(lens),
                                                            num_q_heads, num_kv_heads, min_units))


def kv_paged_attention_prefill_workspace_bytes(total_q: int, num_q_heads: int, head_dim: int,
                                               splits: int) -> int:
    return int(lib.kv_paged_attention_prefill_workspace_bytes(total_q, num_q_heads, head_dim,
                                                              splits))


def kv_paged_attention_prefill_split(out, q, k_pool, v_pool, block_tables, context_lens,
                                     query_start, scale: float, max_query_len: int, splits: int,
                                     workspace, work_items=None, stream=None) -> None:
    """kv_paged_attention_prefill with each block's keys cut into `splits` runs; workspace:
    a device tensor of at least kv_paged_attention_prefill_workspace_bytes bytes."""
    torch = _torch()
    T, Hq, D = q.shape
    NB, Hkv, B, D2 = k_pool.shape
    S = context_lens.numel()
    if D2 != D or tuple(out.shape) != (T, Hq, D) or block_tables.shape[0] != S \
            or query_start.numel() != S + 1 or q.dtype != k_pool.dtype \
            or v_pool.shape != k_pool.shape:
        raise KVError(KV_ERR_INVALID, "kv_paged_attention_prefill_split", "shape/dtype mismatch")
    ws, ws_bytes = (0, 0) if workspace is None else (_dev(workspace, "workspace"),
                                                     workspace.numel() * workspace.element_size())
    _check(lib.kv_paged_attention_prefill_split(
        _dev(out, "out", torch.float32), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), _dev(query_start, "query_start", torch.int32),
        S, T, Hq, Hkv, D, B, NB, float(scale), dtype_code(q), max_query_len,
        None if work_items is None else _dev(work_items, "work_items", torch.int32),
        0 if work_items is None else work_items.shape[0], int(splits), ws, ws_bytes,
        _stream(stream)), "kv_paged_attention_prefill_split")


def kv_paged_attention_prefill_split_fp8(out, q, k_pool, v_pool, block_tables, context_lens,
                                         query_start, scale: float, k_scale: float, v_scale: float,
                                         max_query_len: int, splits: int, workspace,
                                         work_items=None, stream=None) -> None:
    """kv_paged_attention_prefill_split over uint8 E4M3 pools with per-pool scales."""
    torch = _torch()
    T, Hq, D = q.shape
    NB, Hkv, B, D2 = _fp8_pools("kv_paged_attention_prefill_split_fp8", k_pool, v_pool)
    S = context_lens.numel()
    if D2 != D or tuple(out.shape) != (T, Hq, D) or block_tables.shape[0] != S \
            or query_start.numel() != S + 1:
        raise KVError(KV_ERR_INVALID, "kv_paged_attention_prefill_split_fp8", "shape mismatch")
    ws, ws_bytes = (0, 0) if workspace is None else (_dev(workspace, "workspace"),
                                                     workspace.numel() * workspace.element_size())
    _check(lib.kv_paged_attention_prefill_split_fp8(
        _dev(out, "out", torch.float32), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), _dev(query_start, "query_start", torch.int32),
        S, T, Hq, Hkv, D, B, NB, float(scale), dtype_code(q), float(k_scale), float(v_scale),
        max_query_len, None if work_items is None else _dev(work_items, "work_items", torch.int32),
        0 if work_items is None else work_items.shape[0], int(splits), ws, ws_bytes,
        _stream(stream)), "kv_paged_attention_prefill_split_fp8")


def kv_paged_attention_prefill_fp8(out, q, k_pool, v_pool, block_tables, context_lens,
                                   query_start, scale: float, k_scale: float, v_scale: float,
                                   max_query_len: int, work_items=None, stream=None) -> None:
    """kv_paged_attention_prefill over uint8 E4M3 pools with per-pool scales; q f16/bf16."""
    torch = _torch()
    T, Hq, D = q.shape
    NB, Hkv, B, D2 = _fp8_pools("kv_paged_attention_prefill_fp8", k_pool, v_pool)
    S = context_lens.numel()
    if D2 != D or tuple(out.shape) != (T, Hq, D) or block_tables.shape[0] != S \
            or query_start.numel() != S + 1:
        raise KVError(KV_ERR_INVALID, "kv_paged_attention_prefill_fp8", "shape mismatch")
    _check(lib.kv_paged_attention_prefill_fp8(
        _dev(out, "out", torch.float32), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), _dev(query_start, "query_start", torch.int32),
        S, T, Hq, Hkv, D, B, NB, float(scale), dtype_code(q), float(k_scale), float(v_scale),
        max_query_len, None if work_items is None else _dev(work_items, "work_items", torch.int32),
        0 if work_items is None else work_items.shape[0], _stream(stream)),
        "kv_paged_attention_prefill_fp8")
