"""The continuous-batching loop on the oracle's side (test infrastructure).

The same iteration as the pages' scheduling sketch ([P2] "连续批处理：别再等最
慢的那个请求了"), with the readings the library documents, run on
oracle.allocator.AllocatorModel: free finished requests, admit waiting ones
while prompt blocks plus one block per running sequence fit, fork the extra
samples over every prompt block, grow every running sequence by one token with
copy on write, and while that growth does not fit send the latest request back
to the head of the queue (recomputation).

With a swap space of S host slots (a LIFO stack starting [S-1, ..., 0]), a
preempted request that was not admitted in the same iteration and whose
distinct blocks fit in the free slots is swapped out instead: its distinct
blocks, in order of first appearance over its samples' rows, each take a
slot, and the request waits, by request id, in the swapped list. Swapped
requests come back first: at the start of admission, while the first one's
distinct blocks plus one block per running sequence (its own included) are
free, it takes fresh blocks (one alloc), the references its rows hold, and
gives its slots back in order; waiting requests are admitted only when no
request is swapped out.

With a sliding window of W tokens, every iteration after the growth releases
the blocks wholly before each running sequence's last W positions
(AllocatorModel.trim; row entries become -1).
"""

from collections import deque

from oracle import allocator as A

BS = 16


class OracleSeq:
    def __init__(self, rid, sample, row, length, gen_len):
        self.rid, self.sample, self.row = rid, sample, row
        self.length, self.gen_len, self.generated = length, gen_len, 0


def held(s):
    return [b for b in s.row[: -(-s.length // BS)] if b >= 0]


def distinct_blocks(seqs):
    """Distinct block ids over the rows, in order of first appearance, and
    per sequence the index of each row entry in that list (-1: released)."""
    order, index, maps = [], {}, []
    for s in seqs:
        m = []
        for b in s.row[: -(-s.length // BS)]:
            if b < 0:
                m.append(-1)
                continue
            if b not in index:
                index[b] = len(order)
                order.append(b)
            m.append(index[b])
        maps.append(m)
    return order, maps


class OracleBatcher:
    def __init__(self, num_blocks, width, prefix_caching=False, swap_slots=0, window=0):
        self.model = A.AllocatorModel(num_blocks, BS)
        self.width = width
        self.prefix_caching = prefix_caching
        self.waiting = deque()
        self.running = []
        self.specs = {}
        self.swap_free = list(range(swap_slots - 1, -1, -1)) if swap_slots else None
        self.swapped = []   # (rid, seqs, maps, slots), by rid
        self.swap_in = []   # this iteration's (slot, block) pairs
        self.swap_out = []  # this iteration's (block, slot) pairs
        self.swapped_in, self.swapped_out = [], []
        self.window = window
        self.trimmed = 0

    def submit(self, spec):
        self.waiting.append(spec)

    def plan(self):
        m = self.model
        finished, admitted = [], []
        still = []
        for s in self.running:
            if s.generated >= s.gen_len:
                m.free(held(s))
                finished.append((s.rid, s.sample))
            else:
                still.append(s)
        self.running = still
        self.swap_in, self.swap_out, self.swapped_in, self.swapped_out = [], [], [], []
        self.trimmed = 0
        while self.swapped:
            rid, seqs, maps, slots = self.swapped[0]
            if m.num_free() - len(slots) < len(self.running) + len(seqs):
                break
            self.swapped.pop(0)
            ids = m.alloc(len(slots))
            extra = []
            for s, mp in zip(seqs, maps):
                for j, u in enumerate(mp):
                    s.row[j] = ids[u] if u >= 0 else -1
                    if u >= 0:
                        extra.append(ids[u])
            for b in ids:  # one reference came with the alloc
                extra.remove(b)
            m.incref(extra)
            self.swap_in += list(zip(slots, ids))
            self.swap_free.extend(slots)
            self.running.extend(seqs)
            self.swapped_in.append(rid)
        while self.waiting and not self.swapped:
            spec = self.waiting[0]
            need = -(-spec.prompt_len // BS)
            hit = m.acquire(spec.block_keys) if self.prefix_caching else []
            if m.num_free() - (need - len(hit)) < len(self.running) + spec.samples:
                if hit:
                    m.free(hit)
                break
            self.waiting.popleft()
            row = [-1] * self.width
            row[:len(hit)] = hit
            first = len(hit) * BS
            slots = m.extend([row], [first], [spec.prompt_len])
            if self.prefix_caching and len(spec.block_keys) > len(hit):
                m.register(spec.block_keys[len(hit):], row[len(hit):len(spec.block_keys)])
            self.running.append(OracleSeq(spec.rid, 0, row, spec.prompt_len, spec.gen_len))
            for k in range(1, spec.samples):
                r = [-1] * self.width
                m.fork(row, r, need)
                self.running.append(OracleSeq(spec.rid, k, r, spec.prompt_len, spec.gen_len))
            self.specs[spec.rid] = spec
            admitted.append((spec, first, slots))
        slots, copies, preempted = [], [], []
        while self.running:
            rows = [list(s.row) for s in self.running]
            cur = [s.length for s in self.running]
            try:
                slots, copies = m.extend_cow(rows, cur, [c + 1 for c in cur])
            except A.AllocError as e:
                assert e.code == A.OOM
                rid = self.running[-1].rid
                seqs = [s for s in self.running if s.rid == rid]
                order, maps = distinct_blocks(seqs)
                for s in seqs:
                    m.free(held(s))
                self.running = [s for s in self.running if s.rid != rid]
                if (self.swap_free is not None and len(order) <= len(self.swap_free)
                        and all(a[0].rid != rid for a in admitted)):
                    hslots = [self.swap_free.pop() for _ in order]
                    self.swap_out += list(zip(order, hslots))
                    self.swapped.append((rid, seqs, maps, hslots))
                    self.swapped.sort(key=lambda x: x[0])
                    self.swapped_out.append(rid)
                    continue
                # recompute: the latest request goes back to the head of the queue
                admitted = [a for a in admitted if a[0].rid != rid]
                preempted.append(rid)
                self.waiting.appendleft(self.specs[rid])
                continue
            self.trimmed = (m.trim(rows, [c + 1 for c in cur], self.window)
                            if self.window else 0)
            for s, r in zip(self.running, rows):
                s.row = r
                s.length += 1
                s.generated += 1
            break
        batch = list(self.running)
        return finished, admitted, batch, slots, copies, preempted
