"""The continuous-batching loop on the oracle's side (test infrastructure).

The same iteration as the pages' scheduling sketch ([P2] "连续批处理：别再等最
慢的那个请求了"), with the readings the library documents, run on
oracle.allocator.AllocatorModel: free finished requests, admit waiting ones
while prompt blocks plus one block per running sequence fit, fork the extra
samples over every prompt block, grow every running sequence by one token with
copy on write, and while that growth does not fit send the latest request back
to the head of the queue (recomputation).
"""

from collections import deque

from oracle import allocator as A

BS = 16


class OracleSeq:
    def __init__(self, rid, sample, row, length, gen_len):
        self.rid, self.sample, self.row = rid, sample, row
        self.length, self.gen_len, self.generated = length, gen_len, 0


class OracleBatcher:
    def __init__(self, num_blocks, width, prefix_caching=False):
        self.model = A.AllocatorModel(num_blocks, BS)
        self.width = width
        self.prefix_caching = prefix_caching
        self.waiting = deque()
        self.running = []
        self.specs = {}

    def submit(self, spec):
        self.waiting.append(spec)

    def plan(self):
        m = self.model
        finished, admitted = [], []
        still = []
        for s in self.running:
            if s.generated >= s.gen_len:
                m.free(s.row[: -(-s.length // BS)])
                finished.append((s.rid, s.sample))
            else:
                still.append(s)
        self.running = still
        while self.waiting:
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
                # recompute: the latest request goes back to the head of the queue
                rid = self.running[-1].rid
                for s in [s for s in self.running if s.rid == rid]:
                    m.free(s.row[: -(-s.length // BS)])
                self.running = [s for s in self.running if s.rid != rid]
                admitted = [a for a in admitted if a[0].rid != rid]
                preempted.append(rid)
                self.waiting.appendleft(self.specs[rid])
                continue
            for s, r in zip(self.running, rows):
                s.row = r
                s.length += 1
                s.generated += 1
            break
        batch = list(self.running)
        return finished, admitted, batch, slots, copies, preempted
