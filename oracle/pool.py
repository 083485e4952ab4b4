"""KV pool layout, byte sizes and the append step, on the host.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[P2], "PagedAttention：把操作系统的虚拟内存搬进 GPU": the cache memory is cut
into fixed-size physical blocks, and a per-sequence page table maps the
logically contiguous KV of a sequence onto blocks that need not be adjacent;
blocks are handed out as tokens are produced. The pages fix no byte layout;
the one used here is this library's contract:

    element (layer l, c in {K=0, V=1}, block b, kv head h, slot t, dim d)
    lives at element offset ((((l*2 + c)*NB + b)*Hkv + h)*BS + t)*D + d

so one (l, c, b, h) tile of BS x D elements is contiguous and one block id
names the same block in every layer. A swap slot s of host memory holds one
block of every layer, element (l, c, h, t, d) at offset
((((s*L + l)*2 + c)*Hkv + h)*BS + t)*D + d.

[P2], "真正吃显存的是 KV Cache，不是模型权重": per request the cache holds a
K and a V vector per token, per layer and per head; the section works the
product out for a 32-layer, 32-head, head_dim-128 fp16 model at 2048 tokens
(about 1.07 GB per request; 32 concurrent requests take about 34 GB).
"""

import numpy as np

from . import fp8

# Storage element size in bytes per KV dtype name.
ESIZE = {"f16": 2, "bf16": 2, "e4m3": 1}


def kv_bytes_per_request(seq_len: int, layers: int, heads: int, head_dim: int,
                         bytes_per_elem: int) -> int:
    """The pages' closed form: 2 (K and V) x seq x layers x heads x dim x bytes."""
    return 2 * seq_len * layers * heads * head_dim * bytes_per_elem


def pool_shape(num_layers, num_blocks, block_size, num_kv_heads, head_dim):
    return (num_layers, 2, num_blocks, num_kv_heads, block_size, head_dim)


def pool_bytes(num_layers, num_blocks, block_size, num_kv_heads, head_dim, kv_dtype) -> int:
    """Bytes of a pool holding num_blocks blocks in every layer."""
    n = 1
    for s in pool_shape(num_layers, num_blocks, block_size, num_kv_heads, head_dim):
        n *= s
    return n * ESIZE[kv_dtype]


def raw_dtype(kv_dtype):
    return np.uint8 if kv_dtype == "e4m3" else np.uint16


def view_pool(buf: np.ndarray, num_layers, num_blocks, block_size, num_kv_heads,
              head_dim, kv_dtype) -> np.ndarray:
    """View a flat uint8 host copy of the pool as [L, 2, NB, Hkv, BS, D] raw codes."""
    shape = pool_shape(num_layers, num_blocks, block_size, num_kv_heads, head_dim)
    return buf.view(raw_dtype(kv_dtype)).reshape(shape)


def raw_to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of raw fp16 / bf16 bit patterns (uint16)."""
    raw = np.asarray(raw, dtype=np.uint16)
    if dtype == "f16":
        return raw.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        # A bf16 value is the upper half of the fp32 with the same bits.
        return (raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def encode_for_cache(src_raw: np.ndarray, src_dtype: str, kv_dtype: str,
                     scale_per_head=None) -> np.ndarray:
    """Stored codes for source rows [..., Hkv, D] (raw fp16/bf16 bits).

    fp16 / bf16 caches store the source bits unchanged (the source dtype
    must equal the cache dtype). An e4m3 cache stores
    encode(fp32(x / scale[h])) for each kv head h.
    """
    if kv_dtype in ("f16", "bf16"):
        if src_dtype != kv_dtype:
            raise ValueError("a 16-bit cache stores its own dtype")
        return np.asarray(src_raw, dtype=np.uint16).copy()
    x = raw_to_f64(src_raw, src_dtype)
    s = np.asarray(scale_per_head, dtype=np.float32)[:, None]  # [Hkv, 1]
    return fp8.quantize(x, s)


def append(pool6: np.ndarray, layer: int, k_raw: np.ndarray, v_raw: np.ndarray,
           src_dtype: str, kv_dtype: str, slot_mapping, k_scale=None, v_scale=None):
    """Write token t's K and V rows into its slot (in place).

    k_raw, v_raw: [T, Hkv, D] raw source bits. slot_mapping[t] = block * BS + offset;
    a negative slot means "skip this token". Slots in one call are unique.
    """
    block_size = pool6.shape[4]
    k_codes = encode_for_cache(k_raw, src_dtype, kv_dtype, k_scale)
    v_codes = encode_for_cache(v_raw, src_dtype, kv_dtype, v_scale)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    block, offset = np.divmod(slots[keep], block_size)
    # pool6[layer, c, block[t], :, offset[t], :] = codes[t] for every kept t
    pool6[layer, 0, block, :, offset, :] = k_codes[keep]
    pool6[layer, 1, block, :, offset, :] = v_codes[keep]


def copy_blocks(pool6: np.ndarray, src_ids, dst_ids) -> None:
    """Copy on write's copy (in place): every layer's K and V of block
    dst_ids[i] become those of block src_ids[i]. Destinations are distinct
    and none is a source, so the pairs do not depend on one another."""
    src = np.asarray(src_ids, dtype=np.int64)
    dst = np.asarray(dst_ids, dtype=np.int64)
    if src.size:
        pool6[:, :, dst] = pool6[:, :, src]


def swap_out(pool6: np.ndarray, host: np.ndarray, block_ids, host_slots) -> None:
    """Swapping out ("vLLM 也不是银弹：..."): host[slots[i]] := every layer's K
    and V of block ids[i]. host: [S, L, 2, Hkv, BS, D] raw codes, one slot per
    block of the whole model; slots are distinct."""
    ids = np.asarray(block_ids, dtype=np.int64)
    slots = np.asarray(host_slots, dtype=np.int64)
    for b, s in zip(ids, slots):
        host[s] = pool6[:, :, b]


def swap_in(pool6: np.ndarray, host: np.ndarray, host_slots, block_ids) -> None:
    """Swapping in: every layer's K and V of block ids[i] := host[slots[i]];
    blocks are distinct."""
    ids = np.asarray(block_ids, dtype=np.int64)
    slots = np.asarray(host_slots, dtype=np.int64)
    for s, b in zip(slots, ids):
        pool6[:, :, b] = host[s]
