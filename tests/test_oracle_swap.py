"""Pins of the oracle's swap (pool.swap_out / swap_in) and of the loop's swap
preemption (tests/oracle_loop.OracleBatcher with a swap space).

The slot layout is checked element by element against the offset formula of
the layout contract; a swap out and back in to other blocks must equal the
block copy. The loop runs seeded request traces (parallel samples, small
pools) over a pool of token ids: after every iteration's work, applied in the
library's order (swap-ins, swap-outs, prompt writes, block copies, new
tokens), every running sequence must gather exactly its own history, every
swapped-out request's slots must hold its blocks' tokens, and refcounts must
equal the references the rows hold. Planted mistakes (plane order in a slot,
rows rebuilt with the wrong blocks, shared references not restored) fail.
"""

import numpy as np
import pytest

import workloads as W
from oracle import pool as opool
from tests.oracle_loop import OracleBatcher

BS = 16


def test_slot_layout_matches_the_offset_formula():
    L, NB, H, D, S = 3, 5, 2, 4, 3
    p6 = np.arange(L * 2 * NB * H * BS * D, dtype=np.int64).reshape(L, 2, NB, H, BS, D)
    host = np.full((S, L, 2, H, BS, D), -1, dtype=np.int64)
    ids, slots = [4, 0, 2], [1, 2, 0]
    opool.swap_out(p6, host, ids, slots)
    flat_p, flat_h = p6.reshape(-1), host.reshape(-1)
    for b, s in zip(ids, slots):
        for l in range(L):
            for c in range(2):
                for h in range(H):
                    for t in range(BS):
                        for d in range(D):
                            po = ((((l * 2 + c) * NB + b) * H + h) * BS + t) * D + d
                            ho = ((((s * L + l) * 2 + c) * H + h) * BS + t) * D + d
                            assert flat_h[ho] == flat_p[po]


def test_planted_plane_order_fails_the_layout_pin():
    def bad_out(p6, host, ids, slots):
        for b, s in zip(ids, slots):
            host[s] = p6[:, ::-1, b]
    orig = opool.swap_out
    opool.swap_out = bad_out
    try:
        with pytest.raises(AssertionError):
            test_slot_layout_matches_the_offset_formula()
    finally:
        opool.swap_out = orig


def test_round_trip_equals_block_copy():
    rng = np.random.default_rng(1)
    p6 = rng.integers(0, 1 << 16, size=(2, 2, 10, 2, BS, 8)).astype(np.uint16)
    host = np.zeros((4, 2, 2, 2, BS, 8), dtype=np.uint16)
    a, b = p6.copy(), p6.copy()
    opool.swap_out(a, host, [3, 7, 1], [2, 0, 3])
    opool.swap_in(a, host, [2, 0, 3], [5, 8, 9])
    opool.copy_blocks(b, [3, 7, 1], [5, 8, 9])
    assert np.array_equal(a, b)


# ------------------------------------------------------------- the loop ----
def run_trace(batcher_cls, seed, num_blocks, swap_slots, caching=False, window=0):
    groups = (3, 48) if caching else (0, 0)
    trace = W.request_trace("batching_host", seed, 60, max_prompt=60, max_gen=40,
                            prefix_groups=groups[0], shared_tokens=groups[1])
    o = batcher_cls(num_blocks, 7, prefix_caching=caching, swap_slots=swap_slots, window=window)
    tok = np.full(num_blocks * BS, -1, dtype=np.int64)
    host = np.full((max(swap_slots, 1), BS), -1, dtype=np.int64)

    def t_id(rid, sample, pos):
        """Token ids: a full prompt block's are named by its content key (equal
        keys, equal tokens), the rest of the prompt by the request, later
        tokens by the sample."""
        keys = o.specs[rid].block_keys
        if sample < 0 and pos // BS < len(keys):
            return (1 << 50) + ((keys[pos // BS] % (1 << 40)) << 4 | pos % BS)
        return (rid * 8 + (0 if sample < 0 else sample + 1)) * 4096 + pos

    def expected(rid, sample, prompt_len, pos):
        return t_id(rid, -1 if pos < prompt_len else sample, pos)

    pending = list(trace)
    swapped = 0
    for it in range(3000):
        while pending and pending[0].arrival <= it:
            o.submit(pending.pop(0))
        fin, adm, batch, slots, copies, pre = o.plan()
        for s, b in o.swap_in:
            tok[b * BS:(b + 1) * BS] = host[s]
        for b, s in o.swap_out:
            host[s] = tok[b * BS:(b + 1) * BS]
        for spec, first, sl in adm:
            for k, slot in enumerate(sl):
                tok[slot] = t_id(spec.rid, -1, first + k)
        for src, dst in copies:
            tok[dst * BS:(dst + 1) * BS] = tok[src * BS:(src + 1) * BS]
        for s, slot in zip(batch, slots):
            tok[slot] = expected(s.rid, s.sample, o.specs[s.rid].prompt_len, s.length - 1)
        swapped += len(o.swapped_out)
        held = {}
        for s in batch:
            plen = o.specs[s.rid].prompt_len
            lo = max(0, s.length - window) if window else 0
            for pos in range(lo, s.length):
                got = tok[s.row[pos // BS] * BS + pos % BS]
                assert got == expected(s.rid, s.sample, plen, pos), (it, s.rid, s.sample, pos)
            for j, b in enumerate(s.row[: -(-s.length // BS)]):
                if b >= 0:
                    held[b] = held.get(b, 0) + 1
                else:  # only blocks wholly before the window are released
                    assert window and BS * (j + 1) <= s.length - window, (it, s.rid, j)
        for rid, seqs, maps, hs in o.swapped:
            plen = o.specs[rid].prompt_len
            for s, mp in zip(seqs, maps):
                lo = max(0, s.length - window) if window else 0
                for pos in range(lo, s.length):
                    got = host[hs[mp[pos // BS]], pos % BS]
                    assert got == expected(rid, s.sample, plen, pos), (it, rid, pos)
        for b in range(num_blocks):
            assert o.model.ref[b] == held.get(b, 0), (it, b)
        if not pending and not o.running and not o.waiting and not o.swapped:
            break
    assert not o.running and not o.swapped
    return swapped


@pytest.mark.parametrize("seed,num_blocks,swap_slots,caching", [
    (4, 18, 64, False), (12, 18, 8, False), (12, 18, 2, False), (6, 24, 16, True),
    (14, 20, 40, True), (13, 18, 64, False)])
def test_swap_trace_keeps_every_history(seed, num_blocks, swap_slots, caching):
    assert run_trace(OracleBatcher, seed, num_blocks, swap_slots, caching) > 0


@pytest.mark.parametrize("seed,num_blocks,swap_slots,caching,window", [
    (12, 18, 8, False, 33), (12, 14, 32, False, 40), (4, 18, 64, False, 24),
    (6, 24, 16, True, 17), (3, 30, 0, True, 1)])
def test_window_trace_keeps_every_window(seed, num_blocks, swap_slots, caching, window):
    """The loop with a sliding window (blocks before each window released every
    iteration), with swap and prefix caching: every running sequence gathers
    the last W tokens of its history, released entries are only ever wholly
    before the window, refcounts equal the references the rows hold."""
    run_trace(OracleBatcher, seed, num_blocks, swap_slots, caching, window)


def test_planted_eager_trim_fails_the_window_trace():
    class Eager(OracleBatcher):  # releases one block too many
        def plan(self):
            self.window = max(1, self.window - BS)
            try:
                return super().plan()
            finally:
                self.window += BS
    with pytest.raises(AssertionError):
        run_trace(Eager, 12, 18, 8, False, 33)


def test_planted_swap_in_mistakes_fail_the_trace():
    class WrongBlocks(OracleBatcher):
        def plan(self):
            r = super().plan()
            if len(self.swap_in) > 1:  # the data goes to the blocks in reverse order
                s, b = zip(*self.swap_in)
                self.swap_in = list(zip(s, b[::-1]))
            return r

    class NoShare(OracleBatcher):
        def plan(self):  # a request back from swap keeps one reference per distinct block
            r = super().plan()
            for s in [s for s in self.running if s.rid in self.swapped_in and s.sample > 0]:
                for b in s.row[: -(-s.length // BS)]:
                    if self.model.ref[b] > 1:
                        self.model.ref[b] -= 1
            return r

    with pytest.raises(AssertionError):
        run_trace(WrongBlocks, 4, 18, 64)
    with pytest.raises(AssertionError):
        run_trace(NoShare, 4, 18, 64)
