"""Python binding of libpagedkv (paged KV cache + paged decode attention, gfx950).

Argument marshalling only: every step of the hot path runs in the HIP library
(``csrc/``), whose C ABI is ``include/pagedkv.h``. PyTorch tensors supply
device memory and the current stream; host bookkeeping takes numpy arrays.
The functions keep the C names. A non-OK status raises ``PkvError``.

The library must have been built (``python paged_kv_cache_450_amd/build.py``
or ``__graft_entry__.build()``); importing this package fails loudly if it
was not: there is no fallback implementation.
"""

import ctypes
import os

import numpy as np

__all__ = [
    "PKV_OK", "PKV_ERR_INVALID", "PKV_ERR_OOM", "PKV_ERR_STATE", "PKV_ERR_HIP",
    "PKV_F16", "PKV_BF16", "PKV_FP8_E4M3", "BLOCK_SIZE", "PkvError", "PoolDesc",
    "kv_pool_bytes", "kv_pool_create", "kv_pool_destroy", "kv_pool_num_free",
    "kv_pool_free_list", "block_alloc", "block_free", "block_incref", "block_refcount",
    "kv_seq_fork", "kv_seq_extend", "kv_cache_append", "paged_attn_workspace_bytes",
    "paged_attn_decode", "paged_attn_reduce", "pkv_last_error", "library_path", "lib",
    "PrefixPlan", "paged_attn_prefix_plan", "paged_attn_prefix_workspace_bytes",
    "paged_attn_decode_prefix", "paged_attn_decode_prefix_l2", "paged_attn_decode_append_noalloc",
    "STATIC_SCRATCH_BYTES",
]

PKV_OK, PKV_ERR_INVALID, PKV_ERR_OOM, PKV_ERR_STATE, PKV_ERR_HIP = 0, -1, -2, -3, -4
PKV_F16, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2
BLOCK_SIZE = 16
STATIC_SCRATCH_BYTES = 32 << 20  # PKV_STATIC_SCRATCH_BYTES

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpagedkv.so")


def library_path() -> str:
    return _LIB_PATH


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("kv_dtype", ctypes.c_int32)]


def _load():
    # torch ships its own HIP runtime. Load it first so that this library's
    # libamdhip64.so.7 dependency binds to that same runtime: one process must
    # never hold two HIP/HSA runtimes.
    import torch  # noqa: F401

    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python paged_kv_cache_450_amd/build.py` "
            "(there is no fallback path)")
    L = ctypes.CDLL(_LIB_PATH)
    i32, i64, sz, vp, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
    # Host arrays go in as plain addresses (numpy's data pointer as an int):
    # building a typed ctypes pointer per argument costs more than the
    # bookkeeping call itself.
    p_i32 = p_i64 = p_u64 = vp
    p_desc = ctypes.POINTER(PoolDesc)
    sig = {
        "kv_pool_bytes": (sz, [p_desc]),
        "kv_pool_create": (i32, [p_desc, vp, sz, ctypes.POINTER(vp)]),
        "kv_pool_destroy": (None, [vp]),
        "kv_pool_num_free": (i32, [vp]),
        "kv_pool_free_list": (i32, [vp, p_i32, i32]),
        "block_alloc": (i32, [vp, i32, p_i32]),
        "block_free": (i32, [vp, i32, p_i32]),
        "block_incref": (i32, [vp, i32, p_i32]),
        "block_refcount": (i32, [vp, i32]),
        "kv_seq_fork": (i32, [vp, p_i32, p_i32, i32]),
        "kv_seq_extend": (i32, [vp, i32, p_i32, i32, p_i32, p_i32, p_i64]),
        "kv_seq_extend_cow": (i32, [vp, i32, p_i32, i32, p_i32, p_i32, p_i64, p_i32, p_i32,
                                    p_i32]),
        "kv_block_copy": (i32, [vp, p_i32, p_i32, i32, vp]),
        "kv_swap_slot_bytes": (sz, [vp]),
        "kv_swap_out": (i32, [vp, p_i32, p_i32, i32, vp, sz, vp]),
        "kv_swap_in": (i32, [vp, p_i32, p_i32, i32, vp, sz, vp]),
        "kv_prefix_register": (i32, [vp, p_u64, p_i32, i32, p_i32]),
        "kv_prefix_acquire": (i32, [vp, p_u64, i32, p_i32, p_i32]),
        "kv_pool_num_cached": (i32, [vp]),
        "kv_seq_trim": (i32, [vp, i32, p_i32, i32, p_i32, i32, p_i32]),
        "paged_attn_decode_window": (i32, [vp, i32, vp, vp, i32, vp, i32, vp, vp, i32, vp, i32,
                                           i32, f32, vp, vp, i32, i32, vp, sz, i32, vp]),
        "kv_pool_cached_list": (i32, [vp, p_i32, i32]),
        "kv_cache_append": (i32, [vp, i32, vp, vp, i32, vp, i32, vp, vp, vp]),
        "paged_attn_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "paged_attn_decode": (i32, [vp, i32, vp, i32, vp, vp, i32, vp, i32, i32, f32, vp, vp,
                                    i32, i32, vp, sz, vp]),
        "paged_attn_decode_append": (i32, [vp, i32, vp, vp, i32, vp, i32, vp, vp, i32, vp, i32,
                                           i32, f32, vp, vp, i32, i32, vp, sz, vp]),
        "paged_attn_decode_prefix_l2": (i32, [vp, i32, vp, vp, i32, vp, i32, vp, vp, i32, vp,
                                              i32, i32, f32, i32, vp, vp, sz, vp]),
        "paged_attn_decode_append_noalloc": (i32, [vp, i32, vp, vp, i32, vp, i32, vp, vp, i32,
                                                   vp, i32, i32, f32, vp, vp, i32, i32, vp]),
        "paged_attn_reduce": (i32, [vp, vp, i32, vp, i32, i32, i32, i32, i32, vp]),
        "paged_attn_prefix_plan": (i32, [p_i32, i32, p_i32, i32, i32, i32, p_i32, p_i32, p_i32,
                                         p_i32, p_i32, p_i32]),
        "paged_attn_prefix_workspace_bytes": (sz, [i32, i32, i32]),
        "paged_attn_decode_prefix": (i32, [vp, i32, vp, vp, i32, vp, i32, vp, vp, i32, vp, i32,
                                           i32, f32, i32, vp, vp, vp, vp, i32, i32, vp, sz, vp]),
        "pkv_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


lib = _load()


def pkv_last_error() -> str:
    return lib.pkv_last_error().decode()


def _check(status: int) -> None:
    if status != PKV_OK:
        raise PkvError(status, pkv_last_error())


def _i32_ptr(a: np.ndarray) -> int:
    """Address of a host int32 array's data, as the C calls take it."""
    return a.ctypes.data


def _host_i32(a, writable=False) -> np.ndarray:
    arr = np.asarray(a)
    if arr.dtype != np.int32 or not arr.flags.c_contiguous or (writable and not arr.flags.writeable):
        if writable:
            raise ValueError("expected a writable C-contiguous int32 numpy array")
        arr = np.ascontiguousarray(arr, dtype=np.int32)
    return arr


# ----------------------------------------------------------------- pool ----
def kv_pool_bytes(desc: PoolDesc) -> int:
    return int(lib.kv_pool_bytes(ctypes.byref(desc)))


def kv_pool_create(desc: PoolDesc, device_base, nbytes: int):
    """device_base: a device tensor (its data_ptr is used), an int address, or None."""
    base = _ptr(device_base)
    out = ctypes.c_void_p()
    _check(lib.kv_pool_create(ctypes.byref(desc), base, nbytes, ctypes.byref(out)))
    return out


def kv_pool_destroy(pool, _destroy=lib.kv_pool_destroy) -> None:
    # The library function is bound at definition: a pool finalised at
    # interpreter exit may run after this module's globals are cleared.
    _destroy(pool)


def kv_pool_num_free(pool) -> int:
    return int(lib.kv_pool_num_free(pool))


def kv_pool_free_list(pool) -> np.ndarray:
    n = lib.kv_pool_free_list(pool, None, 0)
    if n < 0:
        raise PkvError(PKV_ERR_INVALID, "kv_pool_free_list failed")
    out = np.empty(n, dtype=np.int32)
    lib.kv_pool_free_list(pool, _i32_ptr(out), n)
    return out


def kv_pool_num_cached(pool) -> int:
    return int(lib.kv_pool_num_cached(pool))


def kv_pool_cached_list(pool) -> np.ndarray:
    """Cached blocks (prefix caching), longest cached first."""
    n = lib.kv_pool_cached_list(pool, None, 0)
    if n < 0:
        raise PkvError(PKV_ERR_INVALID, "kv_pool_cached_list failed")
    out = np.empty(n, dtype=np.int32)
    lib.kv_pool_cached_list(pool, _i32_ptr(out), n)
    return out


def _u64_ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def kv_prefix_register(pool, keys, ids) -> int:
    """Register full blocks under content keys; returns how many pairs were taken."""
    k = np.ascontiguousarray(np.asarray(keys, dtype=np.uint64).reshape(-1))
    b = _host_i32(ids).reshape(-1)
    if k.size != b.size:
        raise ValueError("one key per block")
    n = ctypes.c_int32(0)
    _check(lib.kv_prefix_register(pool, _u64_ptr(k), _i32_ptr(b), b.size, ctypes.byref(n)))
    return n.value


def kv_prefix_acquire(pool, keys) -> np.ndarray:
    """Blocks of the longest leading run of registered keys, one reference taken on each."""
    k = np.ascontiguousarray(np.asarray(keys, dtype=np.uint64).reshape(-1))
    out = np.empty(max(k.size, 1), dtype=np.int32)
    m = ctypes.c_int32(0)
    _check(lib.kv_prefix_acquire(pool, _u64_ptr(k), k.size, _i32_ptr(out), ctypes.byref(m)))
    return out[:m.value].copy()


def block_alloc(pool, n: int) -> np.ndarray:
    out = np.empty(max(n, 0), dtype=np.int32)
    _check(lib.block_alloc(pool, n, _i32_ptr(out)))
    return out


def block_free(pool, ids) -> None:
    a = _host_i32(ids).reshape(-1)
    _check(lib.block_free(pool, a.size, _i32_ptr(a)))


def block_incref(pool, ids) -> None:
    a = _host_i32(ids).reshape(-1)
    _check(lib.block_incref(pool, a.size, _i32_ptr(a)))


def block_refcount(pool, block_id: int) -> int:
    return int(lib.block_refcount(pool, block_id))


def kv_seq_fork(pool, src_row, dst_row: np.ndarray, num_blocks: int) -> None:
    src = _host_i32(src_row)
    dst = _host_i32(dst_row, writable=True)
    _check(lib.kv_seq_fork(pool, _i32_ptr(src), _i32_ptr(dst), num_blocks))


def kv_seq_extend(pool, block_tables: np.ndarray, cur_lens, new_lens) -> np.ndarray:
    """Grow sequences; block_tables (int32 [B, W]) is updated in place. Returns slots."""
    bt = _host_i32(block_tables, writable=True)
    if bt.ndim != 2:
        raise ValueError("block_tables must be [num_seqs, max_blocks]")
    cur = _host_i32(cur_lens).reshape(-1)
    new = _host_i32(new_lens).reshape(-1)
    if cur.size != bt.shape[0] or new.size != bt.shape[0]:
        raise ValueError("length arrays do not match block_tables")
    total = int(new.astype(np.int64).sum() - cur.astype(np.int64).sum())
    slots = np.empty(max(total, 0), dtype=np.int64)
    _check(lib.kv_seq_extend(pool, bt.shape[0], _i32_ptr(bt), bt.shape[1], _i32_ptr(cur),
                             _i32_ptr(new), slots.ctypes.data))
    return slots


def kv_seq_extend_cow(pool, block_tables: np.ndarray, cur_lens, new_lens):
    """kv_seq_extend with copy on write. Returns (slots, copy_src, copy_dst): the
    block pairs to copy with kv_block_copy before the new tokens are written."""
    bt = _host_i32(block_tables, writable=True)
    if bt.ndim != 2:
        raise ValueError("block_tables must be [num_seqs, max_blocks]")
    cur = _host_i32(cur_lens).reshape(-1)
    new = _host_i32(new_lens).reshape(-1)
    if cur.size != bt.shape[0] or new.size != bt.shape[0]:
        raise ValueError("length arrays do not match block_tables")
    total = int(new.astype(np.int64).sum() - cur.astype(np.int64).sum())
    slots = np.empty(max(total, 0), dtype=np.int64)
    src = np.empty(max(bt.shape[0], 1), dtype=np.int32)
    dst = np.empty(max(bt.shape[0], 1), dtype=np.int32)
    n = ctypes.c_int32(0)
    _check(lib.kv_seq_extend_cow(pool, bt.shape[0], _i32_ptr(bt), bt.shape[1], _i32_ptr(cur),
                                 _i32_ptr(new),
                                 slots.ctypes.data,
                                 _i32_ptr(src), _i32_ptr(dst), ctypes.byref(n)))
    return slots, src[:n.value].copy(), dst[:n.value].copy()


def kv_seq_trim(pool, block_tables: np.ndarray, context_lens, window: int) -> int:
    """Release the blocks wholly before each sequence's window (entries become
    -1 in place); returns the number of references released."""
    bt = _host_i32(block_tables, writable=True)
    if bt.ndim != 2:
        raise ValueError("block_tables must be [num_seqs, max_blocks]")
    lens = _host_i32(context_lens).reshape(-1)
    if lens.size != bt.shape[0]:
        raise ValueError("one length per table row")
    n = ctypes.c_int32(0)
    _check(lib.kv_seq_trim(pool, bt.shape[0], _i32_ptr(bt), bt.shape[1], _i32_ptr(lens), window,
                           ctypes.byref(n)))
    return n.value


# -------------------------------------------------------------- kernels ----
def _torch():
    import torch
    return torch


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return PKV_F16
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def kv_cache_append(pool, layer: int, k, v, slot_mapping, k_scale=None, v_scale=None,
                    stream=None) -> None:
    """k, v: [T, Hkv, D] fp16/bf16 device tensors; slot_mapping: int64 [T]."""
    torch = _torch()
    _dev(k, "k"); _dev(v, "v"); _dev(slot_mapping, "slot_mapping", torch.int64)
    _dev(k_scale, "k_scale", torch.float32); _dev(v_scale, "v_scale", torch.float32)
    if k.dtype != v.dtype or k.shape != v.shape:
        raise ValueError("k and v must have the same shape and dtype")
    if slot_mapping.numel() != k.shape[0]:
        raise ValueError("one slot per token")
    _check(lib.kv_cache_append(pool, layer, _ptr(k), _ptr(v), _dtype_code(k), _ptr(slot_mapping),
                               k.shape[0], _ptr(k_scale), _ptr(v_scale), _stream(stream)))


def kv_block_copy(pool, src_ids, dst_ids, stream=None) -> None:
    """Copy whole blocks (every layer, K and V) src_ids[i] -> dst_ids[i] (host ids)."""
    src = _host_i32(src_ids).reshape(-1)
    dst = _host_i32(dst_ids).reshape(-1)
    if src.size != dst.size:
        raise ValueError("one destination per source")
    _check(lib.kv_block_copy(pool, _i32_ptr(src), _i32_ptr(dst), src.size, _stream(stream)))


def kv_swap_slot_bytes(pool) -> int:
    """Bytes of one swap slot: one block of every layer, K and V."""
    return int(lib.kv_swap_slot_bytes(pool))


def _swap_buffer(host_buf):
    """(address, bytes) of a swap space: a pinned uint8 CPU tensor, or an
    (address, bytes) pair of pinned host memory."""
    if isinstance(host_buf, tuple):
        return host_buf
    torch = _torch()
    if not isinstance(host_buf, torch.Tensor) or host_buf.device.type != "cpu":
        raise ValueError("host_buf must be a pinned CPU tensor")
    if not host_buf.is_pinned() or not host_buf.is_contiguous():
        raise ValueError("host_buf must be pinned and contiguous")
    return host_buf.data_ptr(), host_buf.numel() * host_buf.element_size()


def kv_swap_out(pool, block_ids, host_slots, host_buf, stream=None) -> None:
    """Swap slot host_slots[i] := block block_ids[i] (host ids), on stream."""
    ids = _host_i32(block_ids).reshape(-1)
    slots = _host_i32(host_slots).reshape(-1)
    if ids.size != slots.size:
        raise ValueError("one slot per block")
    addr, nbytes = _swap_buffer(host_buf)
    _check(lib.kv_swap_out(pool, _i32_ptr(ids), _i32_ptr(slots), ids.size, addr, nbytes,
                           _stream(stream)))


def kv_swap_in(pool, host_slots, block_ids, host_buf, stream=None) -> None:
    """Block block_ids[i] := swap slot host_slots[i] (host ids), on stream."""
    ids = _host_i32(block_ids).reshape(-1)
    slots = _host_i32(host_slots).reshape(-1)
    if ids.size != slots.size:
        raise ValueError("one block per slot")
    addr, nbytes = _swap_buffer(host_buf)
    _check(lib.kv_swap_in(pool, _i32_ptr(slots), _i32_ptr(ids), ids.size, addr, nbytes,
                          _stream(stream)))


def paged_attn_workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int,
                               max_context_len: int, partition_size: int) -> int:
    return int(lib.paged_attn_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len,
                                              partition_size))


def paged_attn_decode(pool, layer: int, q, out, block_tables, context_lens, scale: float,
                      max_context_len: int, partition_size: int = 0, workspace=None,
                      k_scale=None, v_scale=None, stream=None) -> None:
    """q, out: [B, Hq, D]; block_tables int32 [B, W]; context_lens int32 [B] (device)."""
    torch = _torch()
    _dev(q, "q"); _dev(out, "out"); _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32); _dev(workspace, "workspace")
    _dev(k_scale, "k_scale", torch.float32); _dev(v_scale, "v_scale", torch.float32)
    if q.dim() != 3 or block_tables.dim() != 2:
        raise ValueError("q must be [B, Hq, D] and block_tables [B, W]")
    if out is not None and (out.shape != q.shape or out.dtype != q.dtype):
        raise ValueError("out must match q")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.paged_attn_decode(pool, layer, _ptr(q), _dtype_code(q), _ptr(out),
                                 _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                                 q.shape[0], q.shape[1], float(scale), _ptr(k_scale),
                                 _ptr(v_scale), max_context_len, partition_size, _ptr(workspace),
                                 ws_bytes, _stream(stream)))


def paged_attn_decode_append(pool, layer: int, new_k, new_v, q, out, block_tables, context_lens,
                             scale: float, max_context_len: int, partition_size: int = 0,
                             workspace=None, k_scale=None, v_scale=None, stream=None) -> None:
    """The fused decode step: new_k, new_v [B, Hkv, D] (q's dtype) are stored at
    each sequence's last position, then paged_attn_decode runs over them."""
    torch = _torch()
    _dev(new_k, "new_k"); _dev(new_v, "new_v")
    _dev(q, "q"); _dev(out, "out"); _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32); _dev(workspace, "workspace")
    _dev(k_scale, "k_scale", torch.float32); _dev(v_scale, "v_scale", torch.float32)
    if q.dim() != 3 or block_tables.dim() != 2:
        raise ValueError("q must be [B, Hq, D] and block_tables [B, W]")
    if new_k.shape != new_v.shape or new_k.dtype != new_v.dtype or new_k.dim() != 3 or \
            new_k.shape[0] != q.shape[0] or new_k.shape[2] != q.shape[2]:
        raise ValueError("new_k and new_v must be [B, Hkv, D] like q")
    if out is not None and (out.shape != q.shape or out.dtype != q.dtype):
        raise ValueError("out must match q")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.paged_attn_decode_append(
        pool, layer, _ptr(new_k), _ptr(new_v), _dtype_code(new_k), _ptr(q), _dtype_code(q),
        _ptr(out), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), q.shape[0],
        q.shape[1], float(scale), _ptr(k_scale), _ptr(v_scale), max_context_len, partition_size,
        _ptr(workspace), ws_bytes, _stream(stream)))


def paged_attn_decode_append_noalloc(pool, layer: int, new_k, new_v, q, out, block_tables,
                                     context_lens, scale: float, max_context_len: int,
                                     partition_size: int = 0, k_scale=None, v_scale=None,
                                     stream=None) -> None:
    """paged_attn_decode_append with the library's static scratch as its
    workspace (nothing allocated by the caller); out is always written (split-K
    runs its reduce in the same call)."""
    torch = _torch()
    _dev(new_k, "new_k"); _dev(new_v, "new_v")
    _dev(q, "q"); _dev(out, "out"); _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    _dev(k_scale, "k_scale", torch.float32); _dev(v_scale, "v_scale", torch.float32)
    if q.dim() != 3 or block_tables.dim() != 2:
        raise ValueError("q must be [B, Hq, D] and block_tables [B, W]")
    if new_k.shape != new_v.shape or new_k.dtype != new_v.dtype or new_k.dim() != 3 or \
            new_k.shape[0] != q.shape[0] or new_k.shape[2] != q.shape[2]:
        raise ValueError("new_k and new_v must be [B, Hkv, D] like q")
    if out is None or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    _check(lib.paged_attn_decode_append_noalloc(
        pool, layer, _ptr(new_k), _ptr(new_v), _dtype_code(new_k), _ptr(q), _dtype_code(q),
        _ptr(out), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), q.shape[0],
        q.shape[1], float(scale), _ptr(k_scale), _ptr(v_scale), max_context_len, partition_size,
        _stream(stream)))


def paged_attn_decode_window(pool, layer: int, q, out, block_tables, context_lens, scale: float,
                             max_context_len: int, window: int, partition_size: int = 0,
                             workspace=None, k_scale=None, v_scale=None, new_k=None, new_v=None,
                             stream=None) -> None:
    """Sliding-window decode: each sequence attends over its last `window` tokens
    (0: all); with new_k / new_v the step also stores the new tokens."""
    torch = _torch()
    _dev(q, "q"); _dev(out, "out"); _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32); _dev(workspace, "workspace")
    _dev(k_scale, "k_scale", torch.float32); _dev(v_scale, "v_scale", torch.float32)
    _dev(new_k, "new_k"); _dev(new_v, "new_v")
    if q.dim() != 3 or block_tables.dim() != 2:
        raise ValueError("q must be [B, Hq, D] and block_tables [B, W]")
    if out is not None and (out.shape != q.shape or out.dtype != q.dtype):
        raise ValueError("out must match q")
    src = _dtype_code(new_k) if new_k is not None else _dtype_code(q)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.paged_attn_decode_window(
        pool, layer, _ptr(new_k), _ptr(new_v), src, _ptr(q), _dtype_code(q), _ptr(out),
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), q.shape[0], q.shape[1],
        float(scale), _ptr(k_scale), _ptr(v_scale), max_context_len, partition_size,
        _ptr(workspace), ws_bytes, window, _stream(stream)))


def paged_attn_reduce(workspace, out, context_lens, max_context_len: int, partition_size: int,
                      stream=None) -> None:
    """out: [B, Hq, D] fp16/bf16 device tensor."""
    torch = _torch()
    _dev(workspace, "workspace"); _dev(out, "out"); _dev(context_lens, "context_lens", torch.int32)
    _check(lib.paged_attn_reduce(_ptr(workspace), _ptr(out), _dtype_code(out), _ptr(context_lens),
                                 out.shape[0], out.shape[1], out.shape[2], max_context_len,
                                 partition_size, _stream(stream)))


# ------------------------------------------------------- shared prefixes ----
class PrefixPlan:
    """Groups of sequences whose tables begin with the same blocks (host arrays,
    as paged_attn_prefix_plan writes them)."""

    def __init__(self, seq_prefix_blocks, group_offsets, group_members, group_blocks,
                 num_groups: int, max_group_size: int):
        self.seq_prefix_blocks = seq_prefix_blocks
        self.group_offsets = group_offsets
        self.group_members = group_members
        self.group_blocks = group_blocks
        self.num_groups = num_groups
        self.max_group_size = max_group_size

    def groups(self):
        """[(members, blocks)] per group."""
        o = self.group_offsets
        return [(self.group_members[o[k]:o[k + 1]].tolist(), int(self.group_blocks[k]))
                for k in range(self.num_groups)]


def paged_attn_prefix_plan(block_tables, context_lens, max_context_len: int,
                           min_blocks: int = 1) -> PrefixPlan:
    """block_tables: host int32 [B, W]; context_lens: host int32 [B]."""
    bt = _host_i32(block_tables)
    if bt.ndim != 2:
        raise ValueError("block_tables must be [num_seqs, max_blocks]")
    lens = _host_i32(context_lens).reshape(-1)
    n = bt.shape[0]
    if lens.size != n:
        raise ValueError("context_lens does not match block_tables")
    pre = np.zeros(n, dtype=np.int32)
    offs = np.zeros(n + 1, dtype=np.int32)
    mem = np.zeros(max(n, 1), dtype=np.int32)
    blk = np.zeros(max(n, 1), dtype=np.int32)
    ng, mg = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib.paged_attn_prefix_plan(_i32_ptr(bt), bt.shape[1], _i32_ptr(lens), n,
                                      max_context_len, min_blocks, _i32_ptr(pre), _i32_ptr(offs),
                                      _i32_ptr(mem), _i32_ptr(blk), ctypes.byref(ng),
                                      ctypes.byref(mg)))
    k = ng.value
    return PrefixPlan(pre, offs[:k + 1].copy(), mem[:offs[k]].copy(), blk[:k].copy(), k, mg.value)


def paged_attn_prefix_workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int) -> int:
    return int(lib.paged_attn_prefix_workspace_bytes(num_seqs, num_q_heads, head_dim))


def paged_attn_decode_prefix_l2(pool, layer: int, q, out, block_tables, context_lens,
                                scale: float, max_context_len: int, seq_prefix_blocks, workspace,
                                new_k=None, new_v=None, stream=None) -> None:
    """Decode (with new_k / new_v: the fused step) in the balanced pass,
    loading each sequence's shared leading blocks (seq_prefix_blocks, a device
    int32 tensor, or None) with the caching policy so that repeats can hit L2."""
    torch = _torch()
    _dev(q, "q"); _dev(out, "out"); _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32); _dev(workspace, "workspace")
    _dev(new_k, "new_k"); _dev(new_v, "new_v")
    _dev(seq_prefix_blocks, "seq_prefix_blocks", torch.int32)
    if q.dim() != 3 or block_tables.dim() != 2:
        raise ValueError("q must be [B, Hq, D] and block_tables [B, W]")
    if out is None or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if new_k is not None and (new_v is None or new_k.shape != new_v.shape or new_k.dim() != 3 or
                              new_k.shape[0] != q.shape[0] or new_k.shape[2] != q.shape[2]):
        raise ValueError("new_k and new_v must be [B, Hkv, D] like q")
    src = _dtype_code(new_k) if new_k is not None else _dtype_code(q)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.paged_attn_decode_prefix_l2(
        pool, layer, _ptr(new_k), _ptr(new_v), src, _ptr(q), _dtype_code(q), _ptr(out),
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), q.shape[0], q.shape[1],
        float(scale), max_context_len, _ptr(seq_prefix_blocks), _ptr(workspace), ws_bytes,
        _stream(stream)))


def paged_attn_decode_prefix(pool, layer: int, q, out, block_tables, context_lens, scale: float,
                             max_context_len: int, seq_prefix_blocks, group_offsets,
                             group_members, group_blocks, num_groups: int, max_group_size: int,
                             workspace, new_k=None, new_v=None, stream=None) -> None:
    """Decode (with new_k / new_v: the fused step) reading each group's shared
    leading blocks once; the group arrays are device int32 tensors."""
    torch = _torch()
    _dev(q, "q"); _dev(out, "out"); _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32); _dev(workspace, "workspace")
    _dev(new_k, "new_k"); _dev(new_v, "new_v")
    for name, a in (("seq_prefix_blocks", seq_prefix_blocks), ("group_offsets", group_offsets),
                    ("group_members", group_members), ("group_blocks", group_blocks)):
        _dev(a, name, torch.int32)
    if q.dim() != 3 or block_tables.dim() != 2:
        raise ValueError("q must be [B, Hq, D] and block_tables [B, W]")
    if out is None or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if new_k is not None and (new_v is None or new_k.shape != new_v.shape or new_k.dim() != 3 or
                              new_k.shape[0] != q.shape[0] or new_k.shape[2] != q.shape[2]):
        raise ValueError("new_k and new_v must be [B, Hkv, D] like q")
    src = _dtype_code(new_k) if new_k is not None else _dtype_code(q)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.paged_attn_decode_prefix(
        pool, layer, _ptr(new_k), _ptr(new_v), src, _ptr(q), _dtype_code(q), _ptr(out),
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), q.shape[0], q.shape[1],
        float(scale), max_context_len, _ptr(seq_prefix_blocks), _ptr(group_offsets),
        _ptr(group_members), _ptr(group_blocks), num_groups, max_group_size, _ptr(workspace),
        ws_bytes, _stream(stream)))
