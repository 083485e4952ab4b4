"""Host model of the balanced pass's bookkeeping: ranges, head groups, pieces.

The streaming kernel cuts the batch's units (one block of one group of hg kv
heads), ordered (sequence, head group, block), into R equal ranges, one per
group of hg waves; wave i of a group reads head i of every unit of its range.
A run of one context inside a range is a segment: a segment that is the
whole context is written out, otherwise it leaves a piece in the wave's slot
1 (the context begins inside the range) or slot 0. The merge kernel
recomputes, for each context, the ranges wa .. wb that hold its pieces and
the slot of the first one. This model replays both sides in plain Python on
random batches and checks that every tile is read exactly once and that the
merge finds exactly the pieces the streaming side left (no GPU involved)."""

import numpy as np
import pytest


def head_group(num_kv_heads: int, waves_per_workgroup: int) -> int:
    hg = waves_per_workgroup
    while num_kv_heads % hg:
        hg //= 2
    return hg


def streaming_side(tiles, hkv, hg, ranges_cap):
    """Pieces per (sequence, head): [(wave, slot or None when whole, tiles)]."""
    hpg = hkv // hg
    total = sum(tiles) * hpg
    R = min(total, ranges_cap)
    starts = np.concatenate([[0], np.cumsum(np.asarray(tiles, dtype=np.int64) * hpg)])
    pieces, seen = {}, set()
    for k in range(R):
        t0, t1 = total * k // R, total * (k + 1) // R
        assert t1 > t0, "ranges are never empty"
        for gi in range(hg):
            t = t0
            while t < t1:
                s = int(np.searchsorted(starts, t, side="right") - 1)
                nt = tiles[s]
                off = t - starts[s]
                grp, j = off // nt, off % nt
                a_sg = starts[s] + grp * nt  # unit index of the context's first tile
                end = min(t1, a_sg + nt)
                g = grp * hg + gi
                whole = a_sg >= t0 and a_sg + nt <= t1
                pieces.setdefault((s, g), []).append(
                    (k * hg + gi, None if whole else (1 if a_sg > t0 else 0), end - t))
                for jj in range(j, j + end - t):
                    assert (s, g, jj) not in seen
                    seen.add((s, g, jj))
                t = end
    return pieces, seen, total, R


def merge_side(s, g, tiles, hkv, hg, total, R):
    """The (wave, slot) pairs the merge reads for context (s, g), or None when
    one wave wrote it whole."""
    hpg = hkv // hg
    before = sum(tiles[:s])
    nt = tiles[s]
    grp, gi = g // hg, g % hg
    a_sg = before * hpg + grp * nt
    wave_of = lambda t: ((t + 1) * R - 1) // total  # noqa: E731
    wa, wb = wave_of(a_sg), wave_of(a_sg + nt - 1)
    if wa == wb:
        return None, wa * hg + gi
    slot_a = 0 if a_sg <= total * wa // R else 1
    return [(v * hg + gi, slot_a if v == wa else 0) for v in range(wa, wb + 1)], None


@pytest.mark.parametrize("seed", range(6))
def test_every_tile_once_and_merge_finds_every_piece(seed):
    rng = np.random.default_rng(seed)
    for _ in range(400):
        batch = int(rng.integers(1, 40))
        hkv = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 12, 32, 40]))
        wpg = int(rng.choice([4, 8]))
        cap_waves = wpg * int(rng.choice([1, 2, 8, 64, 256]))
        tiles = [int(x) for x in rng.integers(0, 3 if rng.random() < 0.3 else 60, size=batch)]
        if sum(tiles) == 0:
            tiles[0] = 1
        hg = head_group(hkv, wpg)
        pieces, seen, total, R = streaming_side(tiles, hkv, hg, cap_waves // hg)
        assert len(seen) == sum(tiles) * hkv
        slots_used = set()
        for s, nt in enumerate(tiles):
            for g in range(hkv):
                if nt == 0:
                    assert (s, g) not in pieces
                    continue
                got = pieces[(s, g)]
                assert sum(p[2] for p in got) == nt
                expect, whole_wave = merge_side(s, g, tiles, hkv, hg, total, R)
                if expect is None:
                    assert got == [(whole_wave, None, nt)]
                else:
                    assert [(w, slot) for w, slot, _ in got] == expect
                    for w, slot in expect:  # a wave's two slots hold distinct contexts
                        assert (w, slot) not in slots_used
                        slots_used.add((w, slot))
                        assert w < cap_waves


def test_head_groups_follow_the_head_count():
    assert [head_group(h, 8) for h in (1, 2, 3, 4, 6, 8, 12, 32, 40)] == [1, 2, 1, 4, 2, 8, 4, 8, 8]
    assert [head_group(h, 4) for h in (1, 2, 3, 4, 6, 8, 12)] == [1, 2, 1, 4, 2, 4, 4]
