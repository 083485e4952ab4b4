"""Pins of the oracle's sliding-window decode and of the block manager's trim.

Attention: the windowed result must equal textbook softmax attention written
with Python floats over the last W tokens of the logical context, for windows
at and around block boundaries; W >= L must give the unwindowed result bit for
bit; W = 1 must give the last value exactly; blocks wholly before the window
must not be read (their table entries set to -1 and their contents poisoned
leave the result unchanged). Trim: on random grow / fork / trim traces over a
pool of token ids, every sequence must still gather the last W tokens of its
own history, the counts must equal the references held by the tables, and no
block inside a window may be released. Planted mistakes (a window one token
off, a trim one block too eager) must fail these pins.
"""

import math

import numpy as np
import pytest

from oracle import allocator as A
from oracle import attention

BS = 16


def brute_attention(q, k, v, scale, group):
    out = []
    for h in range(len(q)):
        g = h // group
        scores = [scale * sum(a * b for a, b in zip(q[h], k[t][g])) for t in range(len(k))]
        top = max(scores)
        e = [math.exp(s - top) for s in scores]
        tot = sum(e)
        out.append([sum(e[t] * v[t][g][d] for t in range(len(k))) / tot for d in range(len(q[h]))])
    return out


def build(rng, lengths, hkv, dim):
    need = sum(-(-n // BS) for n in lengths)
    num_blocks = need + 3
    pool6 = np.full((1, 2, num_blocks, hkv, BS, dim), 0x7E00, dtype=np.uint16)
    ids = rng.permutation(num_blocks)[:need]
    tables = np.full((len(lengths), max(-(-n // BS) for n in lengths) + 1), -1, dtype=np.int32)
    ks, vs, pos = [], [], 0
    for i, n in enumerate(lengths):
        k = rng.standard_normal((n, hkv, dim)).astype(np.float16).view(np.uint16)
        v = rng.standard_normal((n, hkv, dim)).astype(np.float16).view(np.uint16)
        ks.append(k)
        vs.append(v)
        for j in range(-(-n // BS)):
            b = int(ids[pos]); pos += 1
            tables[i, j] = b
            lo, hi = j * BS, min((j + 1) * BS, n)
            pool6[0, 0, b, :, : hi - lo] = k[lo:hi].transpose(1, 0, 2)
            pool6[0, 1, b, :, : hi - lo] = v[lo:hi].transpose(1, 0, 2)
    return pool6, tables, ks, vs


def f64(raw):
    return raw.view(np.float16).astype(np.float64)


LENGTHS = [1, 15, 16, 17, 31, 32, 33, 50, 64, 70]


def check_window(decode_fn, seed=0):
    rng = np.random.default_rng(seed)
    for hq, hkv, dim in [(2, 2, 8), (4, 1, 4)]:
        pool6, tables, ks, vs = build(rng, LENGTHS, hkv, dim)
        q = rng.standard_normal((len(LENGTHS), hq, dim))
        for w in (1, 2, 15, 16, 17, 33, 48):
            got = decode_fn(pool6, 0, q, tables, np.array(LENGTHS), 0.4, "f16", window=w)
            for i, n in enumerate(LENGTHS):
                lo = max(0, n - w)
                ref = brute_attention(q[i].tolist(), f64(ks[i][lo:]).tolist(),
                                      f64(vs[i][lo:]).tolist(), 0.4, hq // hkv)
                assert np.allclose(got[i], ref, rtol=1e-12, atol=1e-12), (w, n)


def test_window_matches_brute_force_on_the_last_w_tokens():
    check_window(attention.paged_decode)


def test_window_at_least_length_is_the_full_context_bitwise():
    rng = np.random.default_rng(2)
    pool6, tables, _, _ = build(rng, LENGTHS, 2, 8)
    q = rng.standard_normal((len(LENGTHS), 4, 8))
    full = attention.paged_decode(pool6, 0, q, tables, np.array(LENGTHS), 0.3, "f16")
    for w in (70, 71, 1000):
        got = attention.paged_decode(pool6, 0, q, tables, np.array(LENGTHS), 0.3, "f16", window=w)
        assert np.array_equal(got, full)


def test_window_of_one_gives_the_last_value_exactly():
    rng = np.random.default_rng(3)
    pool6, tables, _, vs = build(rng, LENGTHS, 2, 8)
    q = rng.standard_normal((len(LENGTHS), 2, 8)) * 20
    got = attention.paged_decode(pool6, 0, q, tables, np.array(LENGTHS), 1.0, "f16", window=1)
    for i, n in enumerate(LENGTHS):
        assert np.array_equal(got[i], f64(vs[i])[n - 1])


def test_blocks_before_the_window_are_not_read():
    rng = np.random.default_rng(4)
    pool6, tables, _, _ = build(rng, LENGTHS, 2, 8)
    q = rng.standard_normal((len(LENGTHS), 2, 8))
    w = 17
    ref = attention.paged_decode(pool6, 0, q, tables, np.array(LENGTHS), 0.5, "f16", window=w)
    poisoned, cut = pool6.copy(), tables.copy()
    for i, n in enumerate(LENGTHS):
        for j in range(max(0, n - w) // BS):
            poisoned[0, :, cut[i, j]] = 0x7E00
            cut[i, j] = -1
    got = attention.paged_decode(poisoned, 0, q, cut, np.array(LENGTHS), 0.5, "f16", window=w)
    assert np.array_equal(got, ref)


def test_planted_window_mistakes_fail_brute_force():
    def shifted(delta):
        def decode(pool6, layer, q, tables, lens, scale, kv_dtype, window=0):
            out = np.zeros(q.shape)
            for i, n in enumerate(lens):
                lo = min(max(0, int(n) - window + delta), int(n) - 1)
                kr, vr = attention.gather_range(pool6, layer, tables[i], lo, int(n))
                out[i] = attention.attend(q[i], f64(kr), f64(vr), scale)
            return out
        return decode
    for delta in (-1, 1):
        with pytest.raises(AssertionError):
            check_window(shifted(delta))


# ------------------------------------------------------------------ trim ----
def trace(model, seed, window, steps=200, num_blocks=48, width=12):
    """Random grow / fork / finish / trim trace; every slot of the pool holds
    the token id written there. Returns the number of blocks trimmed."""
    rng = np.random.default_rng(seed)
    slots = np.full(num_blocks * BS, -1, dtype=np.int64)
    seqs = {}  # id -> (row, history)
    nid, trimmed = 0, 0
    for _ in range(steps):
        op = rng.random()
        if op < 0.15 and seqs:
            r = list(seqs)[int(rng.integers(0, len(seqs)))]
            model.free([b for b in seqs[r][0] if b >= 0])
            del seqs[r]
        elif op < 0.25 and seqs:
            r = list(seqs)[int(rng.integers(0, len(seqs)))]
            row, hist = seqs[r]
            n = len(hist)
            if n % BS == 0 and n > 0:  # fork only at block boundaries: no copy needed
                dst = [-1] * width
                nb = -(-n // BS)
                live = [j for j in range(nb) if row[j] >= 0]
                model.incref([row[j] for j in live])
                for j in live:
                    dst[j] = row[j]
                seqs[nid] = (dst, list(hist)); nid += 1
        elif op < 0.4:
            seqs[nid] = ([-1] * width, []); nid += 1
        else:
            for r in list(seqs):
                row, hist = seqs[r]
                n = len(hist)
                grow = int(rng.integers(1, 6))
                if -(-(n + grow) // BS) > width:
                    continue
                if n % BS and model.refcount(row[n // BS]) > 1:
                    continue
                try:
                    new = model.extend([row], [n], [n + grow])
                except A.AllocError:
                    continue
                for s in new:
                    tok = int(rng.integers(0, 1 << 40))
                    slots[s] = tok
                    hist.append(tok)
        rows = list(seqs)
        if rows:
            tabs = [seqs[r][0] for r in rows]
            lens = [len(seqs[r][1]) for r in rows]
            trimmed += model.trim(tabs, lens, window)
        held = {}
        for r, (row, hist) in seqs.items():
            n = len(hist)
            lo = max(0, n - window)
            for j in range(lo // BS, -(-n // BS)):
                assert row[j] >= 0, (r, j)
            for p in range(lo, n):
                assert slots[row[p // BS] * BS + p % BS] == hist[p], (r, p)
            for b in row:
                if b >= 0:
                    held[b] = held.get(b, 0) + 1
        for b in range(num_blocks):
            assert model.refcount(b) == held.get(b, 0), b
    return trimmed


@pytest.mark.parametrize("window", [1, 16, 17, 40])
def test_trim_keeps_every_window_and_the_counts(window):
    trimmed = sum(trace(A.AllocatorModel(48, BS), seed, window) for seed in range(4))
    assert trimmed > 20


def test_trim_validates_before_changing_anything():
    m = A.AllocatorModel(8, BS)
    row = m.alloc(3) + [-1]
    with pytest.raises(A.AllocError) as e:
        m.trim([list(row)], [48], 0)
    assert e.value.code == A.INVALID
    bad = [row[0], 99, row[2], -1]
    with pytest.raises(A.AllocError) as e:
        m.trim([bad], [48], 1)
    assert e.value.code == A.INVALID and m.refcount(row[0]) == 1
    # The same block listed by two rows but held once: STATE, nothing released.
    with pytest.raises(A.AllocError) as e:
        m.trim([list(row), list(row)], [48, 48], 1)
    assert e.value.code == A.STATE and m.num_free() == 5
    t = [list(row)]
    assert m.trim(t, [48], 16) == 2 and t[0] == [-1, -1, row[2], -1] and m.num_free() == 7
    assert m.trim(t, [48], 16) == 0


def test_planted_eager_trim_fails_the_trace():
    class Eager(A.AllocatorModel):
        def trim(self, tables, lens, window):
            return super().trim(tables, lens, max(1, window - BS))
    with pytest.raises(AssertionError):
        for seed in range(4):
            trace(Eager(48, BS), seed, 17)
