"""Single-query decode attention over a paged KV cache, in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[P2], "PagedAttention：把操作系统的虚拟内存搬进 GPU": the attention kernel reads
each sequence's K and V from non-contiguous physical blocks through the page
table. Paging moves bytes; it does not change the result. So the oracle is
the plain definition of attention on the gathered, logically contiguous K/V:

    s_t = scale * <q_h, k_t>,  p = exp(s - max s),  o_h = (p @ V) / sum(p)

for every query head h, with kv head g = h // (Hq / Hkv) (contiguous query
head groups share one kv head; reading taken where the pages are silent).

Sliding window ([P2] "vLLM 也不是银弹：...", third pitfall, names it as a
long-context remedy; the form is the usual one, reading taken): with a window
of W tokens a sequence of length L attends over positions [max(0, L - W), L)
only, i.e. the same definition on the last W tokens; the blocks wholly before
them are not read at all (their table entries may be gone).

Split-K (not on the pages; the long-context path of this library): the
context is cut into partitions of PS tokens; partition p covers tokens
[p*PS, min((p+1)*PS, L)) and yields m_p = max s, l_p = sum exp(s - m_p) and
o_p = sum exp(s - m_p) v / l_p. Merging uses M = max m_p, w_p = l_p exp(m_p - M),
o = sum w_p o_p / sum w_p, which is exact in real arithmetic.
"""

import numpy as np

from . import fp8
from .pool import raw_to_f64


def kv_to_f64(raw: np.ndarray, kv_dtype: str, scale_per_head=None) -> np.ndarray:
    """Exact float64 values of stored K or V codes shaped [..., Hkv, D]."""
    if kv_dtype == "e4m3":
        s = np.asarray(scale_per_head, dtype=np.float32)[:, None]
        return fp8.dequantize(raw, s)
    return raw_to_f64(raw, kv_dtype)


def gather(pool6: np.ndarray, layer: int, table_row, context_len: int):
    """Raw K and V of one sequence in logical order: two [L, Hkv, D] arrays.

    Reads ceil(L / BS) ids from the sequence's block table and keeps the first
    L slots; entries of the table past those ids are never read.
    """
    block_size = pool6.shape[4]
    n_blocks = -(-context_len // block_size)
    ids = np.asarray(table_row[:n_blocks], dtype=np.int64)
    out = []
    for c in (0, 1):
        tiles = pool6[layer, c, ids]  # [nb, Hkv, BS, D]
        seq = tiles.transpose(0, 2, 1, 3).reshape(n_blocks * block_size,
                                                  tiles.shape[1], tiles.shape[3])
        out.append(seq[:context_len])
    return out[0], out[1]


def gather_range(pool6: np.ndarray, layer: int, table_row, lo: int, hi: int):
    """Raw K and V of positions [lo, hi) of one sequence: two [hi - lo, Hkv, D]
    arrays. Reads only the ids of blocks lo // BS .. ceil(hi / BS) - 1."""
    block_size = pool6.shape[4]
    j0, j1 = lo // block_size, -(-hi // block_size)
    ids = np.asarray(table_row[j0:j1], dtype=np.int64)
    out = []
    for c in (0, 1):
        tiles = pool6[layer, c, ids]  # [nb, Hkv, BS, D]
        seq = tiles.transpose(0, 2, 1, 3).reshape(ids.size * block_size,
                                                  tiles.shape[1], tiles.shape[3])
        out.append(seq[lo - j0 * block_size: hi - j0 * block_size])
    return out[0], out[1]


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q K^T) V per query head.

    q: [Hq, D], k and v: [L, Hkv, D], all float64. Returns [Hq, D].
    """
    num_q_heads = q.shape[0]
    num_kv_heads = k.shape[1]
    group = num_q_heads // num_kv_heads
    out = np.zeros_like(q)
    if k.shape[0] == 0:
        return out
    for h in range(num_q_heads):
        g = h // group
        s = (k[:, g, :] @ q[h]) * scale
        p = np.exp(s - s.max())
        out[h] = (p @ v[:, g, :]) / p.sum()
    return out


def paged_decode(pool6, layer, q_f64, block_tables, context_lens, scale, kv_dtype,
                 k_scale=None, v_scale=None, window: int = 0) -> np.ndarray:
    """Decode attention for a batch: out[i] = attend(q[i], K_i, V_i) in float64.

    q_f64: [B, Hq, D] float64. block_tables: [B, max_blocks] ints.
    context_lens: [B]; a sequence of length 0 gives zeros. window > 0: each
    sequence attends over its last `window` positions only.
    """
    num_seqs = q_f64.shape[0]
    out = np.zeros(q_f64.shape, dtype=np.float64)
    for i in range(num_seqs):
        length = int(context_lens[i])
        if window > 0:
            k_raw, v_raw = gather_range(pool6, layer, block_tables[i], max(0, length - window),
                                        length)
        else:
            k_raw, v_raw = gather(pool6, layer, block_tables[i], length)
        k = kv_to_f64(k_raw, kv_dtype, k_scale)
        v = kv_to_f64(v_raw, kv_dtype, v_scale)
        out[i] = attend(q_f64[i], k, v, scale)
    return out


def partials(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, partition_size: int):
    """Per-partition (m, l, o) of one sequence: [P, Hq], [P, Hq], [P, Hq, D]."""
    length = k.shape[0]
    num_parts = -(-length // partition_size)
    num_q_heads, dim = q.shape
    group = num_q_heads // k.shape[1]
    m = np.full((num_parts, num_q_heads), -np.inf)
    l = np.zeros((num_parts, num_q_heads))
    o = np.zeros((num_parts, num_q_heads, dim))
    for p in range(num_parts):
        lo, hi = p * partition_size, min((p + 1) * partition_size, length)
        for h in range(num_q_heads):
            g = h // group
            s = (k[lo:hi, g, :] @ q[h]) * scale
            m[p, h] = s.max()
            e = np.exp(s - m[p, h])
            l[p, h] = e.sum()
            o[p, h] = (e @ v[lo:hi, g, :]) / l[p, h]
    return m, l, o


def merge(m: np.ndarray, l: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Combine partition partials [P, Hq], [P, Hq], [P, Hq, D] into [Hq, D].

    Zero partitions give zeros.
    """
    if m.shape[0] == 0:
        return np.zeros(o.shape[1:])
    big_m = m.max(axis=0)
    w = l * np.exp(m - big_m)
    return (w[:, :, None] * o).sum(axis=0) / w.sum(axis=0)[:, None]
