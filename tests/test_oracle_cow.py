"""Pins of the oracle's copy on write (AllocatorModel.extend_cow and
pool.copy_blocks).

[P2] "PagedAttention：把操作系统的虚拟内存搬进 GPU": one physical block may
back logical blocks of several sequences (beam search, shared prompts). A
sequence must then see exactly the tokens it was given, whatever the others
sharing its blocks write later. The traces below fork sequences at arbitrary
lengths (so the partially filled last block is shared too), grow them, free
them, and after every step gather each live sequence's tokens through its
table from a pool of token labels: the result must be the sequence's own
history. A copy that is skipped, reversed or not taken, or a reference that is
not released, breaks that or the refcount invariant; the planted mistakes at
the end check that it does.
"""

import numpy as np
import pytest

from oracle import allocator as A
from oracle import pool as opool

BS = 16
WIDTH = 12  # blocks per table row


def invariants(m, tables):
    held = {}
    for row in tables.values():
        for b in row:
            if b >= 0:
                held[b] = held.get(b, 0) + 1
    for b in range(m.num_blocks):
        assert m.ref[b] == held.get(b, 0), b
    assert sorted(m.free_stack) == [b for b in range(m.num_blocks) if m.ref[b] == 0]


def gather(pool6, row, length):
    """Token labels of positions 0..length-1 through a table row (K plane)."""
    return [int(pool6[0, 0, row[p // BS], 0, p % BS, 0]) for p in range(length)]


def run(model_cls, seed, num_blocks=48, steps=250):
    rng = np.random.default_rng(seed)
    m = model_cls(num_blocks, BS)
    pool6 = np.full((1, 2, num_blocks, 1, BS, 1), -1, dtype=np.int64)
    tables, hist = {}, {}
    next_label, next_id = 1, 0
    copies_seen = 0
    for _ in range(steps):
        op = rng.random()
        if op < 0.15 and tables:  # finish a sequence
            r = list(tables)[int(rng.integers(0, len(tables)))]
            m.free([b for b in tables[r] if b >= 0])
            del tables[r], hist[r]
        elif op < 0.35 and tables:  # fork: share every block, the partial one too
            src = list(tables)[int(rng.integers(0, len(tables)))]
            nb = -(-len(hist[src]) // BS)
            row = [-1] * WIDTH
            m.fork(tables[src], row, nb)
            tables[next_id], hist[next_id] = row, list(hist[src])
            next_id += 1
        elif op < 0.45:  # admit a new sequence with a prompt
            row = [-1] * WIDTH
            plen = int(rng.integers(1, 40))
            try:
                slots, copies = m.extend_cow([row], [0], [plen])
            except A.AllocError as e:
                assert e.code == A.OOM
                continue
            assert copies == []
            labels = list(range(next_label, next_label + plen))
            next_label += plen
            for s, lab in zip(slots, labels):
                pool6[0, 0, s // BS, 0, s % BS, 0] = lab
                pool6[0, 1, s // BS, 0, s % BS, 0] = -lab
            tables[next_id], hist[next_id] = row, labels
            next_id += 1
        elif tables:  # grow a random subset by 1..3 tokens in one call
            rids = [r for r in tables if rng.random() < 0.6] or [list(tables)[0]]
            cur = [len(hist[r]) for r in rids]
            new = [min(c + int(rng.integers(1, 4)), WIDTH * BS) for c in cur]
            rows = [tables[r] for r in rids]
            before = (list(m.free_stack), list(m.ref), [list(r) for r in rows])
            try:
                slots, copies = m.extend_cow(rows, cur, new)
            except A.AllocError as e:
                assert e.code == A.OOM
                assert (m.free_stack, m.ref, [list(r) for r in rows]) == before
                continue
            copies_seen += len(copies)
            if copies:
                src, dst = zip(*copies)
                assert len(set(dst)) == len(dst) and not set(dst) & set(src)
                opool.copy_blocks(pool6, list(src), list(dst))
            k = 0
            for r, c, n in zip(rids, cur, new):
                for p in range(c, n):
                    lab = next_label
                    next_label += 1
                    s = slots[k]
                    k += 1
                    assert s // BS == tables[r][p // BS]
                    pool6[0, 0, s // BS, 0, s % BS, 0] = lab
                    pool6[0, 1, s // BS, 0, s % BS, 0] = -lab
                    hist[r].append(lab)
        invariants(m, tables)
        for r in tables:
            got = gather(pool6, tables[r], len(hist[r]))
            assert got == hist[r], (r, got, hist[r])
            assert [-int(pool6[0, 1, tables[r][p // BS], 0, p % BS, 0])
                    for p in range(len(hist[r]))] == hist[r]
    return copies_seen


@pytest.mark.parametrize("seed", range(8))
def test_every_sequence_keeps_its_own_tokens(seed):
    assert run(A.AllocatorModel, seed) > 0  # the traces do exercise copy on write


def test_last_of_the_sharers_keeps_the_block():
    m = A.AllocatorModel(8, BS)
    a = [-1] * 2
    m.extend_cow([a], [0], [5])
    b, c = [-1] * 2, [-1] * 2
    m.fork(a, b, 1)
    m.fork(a, c, 1)
    shared = a[0]
    assert m.ref[shared] == 3
    slots, copies = m.extend_cow([a, b, c], [5, 5, 5], [6, 6, 6])
    assert [s for s, _ in copies] == [shared, shared]
    assert c[0] == shared and a[0] != shared and b[0] != shared
    assert m.ref[shared] == 1 and m.ref[a[0]] == 1 and m.ref[b[0]] == 1
    assert slots == [a[0] * BS + 5, b[0] * BS + 5, shared * BS + 5]


def test_a_full_shared_block_is_not_copied():
    m = A.AllocatorModel(8, BS)
    a = [-1] * 3
    m.extend_cow([a], [0], [BS])
    b = [-1] * 3
    m.fork(a, b, 1)
    slots, copies = m.extend_cow([b], [BS], [BS + 1])
    assert copies == [] and b[0] == a[0] and m.ref[a[0]] == 2
    assert slots == [b[1] * BS]


def test_copies_count_against_free_blocks():
    m = A.AllocatorModel(3, BS)
    a = [-1] * 2
    m.extend_cow([a], [0], [5])
    b = [-1] * 2
    m.fork(a, b, 1)
    m.alloc(1)  # one free block left
    state = (list(m.free_stack), list(m.ref), list(a), list(b))
    with pytest.raises(A.AllocError) as e:  # copy for a, copy-free write for b, and a new block
        m.extend_cow([a, b], [5, 5], [6, BS + 1])
    assert e.value.code == A.OOM
    assert (m.free_stack, m.ref, a, b) == state
    slots, copies = m.extend_cow([a, b], [5, 5], [6, 6])  # exactly one copy fits
    assert len(copies) == 1 and m.num_free() == 0


def test_copy_blocks_moves_every_layer_and_plane():
    p = np.arange(3 * 2 * 5 * 2 * BS * 4).reshape(3, 2, 5, 2, BS, 4)
    before = p.copy()
    opool.copy_blocks(p, [1, 1, 4], [0, 2, 3])
    for d, s in ((0, 1), (2, 1), (3, 4)):
        assert np.array_equal(p[:, :, d], before[:, :, s])
    assert np.array_equal(p[:, :, 1], before[:, :, 1]) and np.array_equal(p[:, :, 4], before[:, :, 4])


# -- planted mistakes: each must break the pin ---------------------------------
class NoCopy(A.AllocatorModel):
    """Writes into the shared block (no copy on write)."""
    def extend_cow(self, tables, cur_lens, new_lens):
        saved = list(self.ref)
        for i, row in enumerate(tables):
            c = int(cur_lens[i])
            if new_lens[i] > c and c % BS:
                self.ref[int(row[c // BS])] = 1
        try:
            slots, _ = self._extend(tables, cur_lens, new_lens, cow=True)
        finally:
            for b in range(self.num_blocks):
                if saved[b] > 1:
                    self.ref[b] = saved[b]
        return slots, []


class KeepsReference(A.AllocatorModel):
    """Takes the copy but never releases the shared block."""
    def extend_cow(self, tables, cur_lens, new_lens):
        slots, copies = self._extend(tables, cur_lens, new_lens, cow=True)
        for s, _ in copies:
            self.ref[s] += 1
        return slots, copies


class ReversedCopy(A.AllocatorModel):
    """Reports the pair backwards (fresh block copied over the shared one)."""
    def extend_cow(self, tables, cur_lens, new_lens):
        slots, copies = self._extend(tables, cur_lens, new_lens, cow=True)
        return slots, [(d, s) for s, d in copies]


@pytest.mark.parametrize("bad", [NoCopy, KeepsReference, ReversedCopy])
def test_planted_mistakes_fail(bad):
    failed = 0
    for seed in range(8):
        try:
            run(bad, seed)
        except (AssertionError, A.AllocError):
            failed += 1
    assert failed > 0
