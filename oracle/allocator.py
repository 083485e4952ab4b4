"""Reference model of the refcounted block manager and slot bookkeeping.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix ([P2]):

* "PagedAttention：把操作系统的虚拟内存搬进 GPU": blocks have one fixed size,
  are handed out on demand as tokens are generated (so a sequence of length L
  holds ceil(L / BS) blocks), suffer no external fragmentation (any free block
  serves any request, so a request for n blocks can succeed exactly when n are
  free), and one physical block may back logical blocks of several sequences
  (beam search, shared prompt prefixes / prefix caching).
* "连续批处理：别再等最慢的那个请求了": every scheduler iteration frees the
  block tables of finished requests, reads the number of free blocks, admits
  waiting requests while they can be allocated, then runs one decode step.

What the pages leave open, and the reading taken (this library's policy):

* free ids sit on a LIFO stack that starts as [N-1, ..., 1, 0], so the first
  allocations return 0, 1, 2, ...; alloc pops, a block whose count reaches 0 is
  pushed back in argument order;
* sharing is a reference count per block: alloc sets it to 1, incref adds 1,
  free subtracts 1;
* every call validates all of its arguments before it changes anything, and
  fails as a whole: INVALID (bad argument), OOM (too few free blocks), STATE
  (freeing a free block, sharing a free block, appending into a block that is
  shared - unless the call is the copy-on-write form);
* copy on write (``extend_cow``): a sequence whose next token lands in a
  partially filled block that other rows still hold first takes a fresh
  block, which must receive a copy of the shared one before the token is
  written; it releases its reference on the shared block. Sequences are
  served in index order, so of k rows sharing a block the first k - 1 writers
  copy and the last one keeps the original;
* a sequence grows one token at a time: the token at position pos goes to slot
  table[pos // BS] * BS + pos % BS, and a new block is taken from the stack
  when pos % BS == 0; sequences of one call are served in index order.

Prefix caching ("PagedAttention：...": requests sharing a prompt prefix share
its blocks; "从零开始：..." step three), with the reading taken:

* the caller names a full block's contents with a key; a block keeps the
  first key it gets, a key the first block;
* a keyed block whose count reaches 0 keeps its contents and joins the back
  of a cached list instead of the free stack; looking its key up revives it;
* allocation takes the free stack first, then the front of the cached list
  (the longest cached block), whose key is dropped; cached blocks count as
  free.
"""

OK, INVALID, OOM, STATE = 0, -1, -2, -3


class AllocError(Exception):
    def __init__(self, code, msg):
        super().__init__(msg)
        self.code = code


class AllocatorModel:
    def __init__(self, num_blocks: int, block_size: int = 16):
        if num_blocks < 0 or block_size <= 0:
            raise AllocError(INVALID, "bad pool size")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free_stack = list(range(num_blocks - 1, -1, -1))
        self.ref = [0] * num_blocks
        self.key_of = {}      # block -> key
        self.block_of = {}    # key -> block
        self.cached = []      # keyed blocks with no reference, oldest first

    # -- block manager -------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free_stack) + len(self.cached)

    def _take(self) -> int:
        if self.free_stack:
            b = self.free_stack.pop()
        else:
            b = self.cached.pop(0)
            del self.block_of[self.key_of.pop(b)]
        self.ref[b] = 1
        return b

    def _release(self, b) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.key_of:
                self.cached.append(b)
            else:
                self.free_stack.append(b)

    def refcount(self, block_id: int) -> int:
        if 0 <= block_id < self.num_blocks:
            return self.ref[block_id]
        return -1

    def alloc(self, n: int) -> list:
        if n < 0:
            raise AllocError(INVALID, "negative count")
        if n > self.num_free():
            raise AllocError(OOM, "not enough free blocks")
        return [self._take() for _ in range(n)]

    def _check_ids(self, ids):
        for b in ids:
            if not 0 <= b < self.num_blocks:
                raise AllocError(INVALID, "block id out of range")

    def free(self, ids) -> None:
        ids = [int(b) for b in ids]
        self._check_ids(ids)
        need = {}
        for b in ids:
            need[b] = need.get(b, 0) + 1
        for b, c in need.items():
            if self.ref[b] < c:
                raise AllocError(STATE, "freeing a block more times than it is held")
        for b in ids:
            self._release(b)

    def incref(self, ids) -> None:
        ids = [int(b) for b in ids]
        self._check_ids(ids)
        for b in ids:
            if self.ref[b] == 0:
                raise AllocError(STATE, "sharing a free block")
        for b in ids:
            self.ref[b] += 1

    # -- per-sequence bookkeeping -------------------------------------------
    def fork(self, src_row, dst_row, n_blocks: int) -> None:
        """dst_row[:n] = src_row[:n] and take one more reference on each id."""
        if n_blocks < 0 or n_blocks > len(src_row) or n_blocks > len(dst_row):
            raise AllocError(INVALID, "bad block count")
        ids = [int(b) for b in src_row[:n_blocks]]
        self.incref(ids)
        for j, b in enumerate(ids):
            dst_row[j] = b

    def extend(self, tables, cur_lens, new_lens) -> list:
        """Grow sequence i from cur_lens[i] to new_lens[i] tokens.

        tables: list of mutable rows (one per sequence, all of the same width).
        Returns the slots of the new tokens, sequence by sequence, in position
        order. Fails as a whole (INVALID, STATE or OOM) with nothing changed.
        """
        return self._extend(tables, cur_lens, new_lens, cow=False)[0]

    def extend_cow(self, tables, cur_lens, new_lens):
        """extend with copy on write. Returns (slots, copies): copies lists the
        (shared block, fresh block) pairs in the order they were taken."""
        return self._extend(tables, cur_lens, new_lens, cow=True)

    def _extend(self, tables, cur_lens, new_lens, cow):
        bs = self.block_size
        num_seqs = len(tables)
        if len(cur_lens) != num_seqs or len(new_lens) != num_seqs:
            raise AllocError(INVALID, "length arrays do not match")
        # Validation walks the sequences in order on a scratch copy of the
        # counts, so that it sees the copies taken by earlier sequences.
        ref = list(self.ref)
        needed = 0
        for i in range(num_seqs):
            cur, new = int(cur_lens[i]), int(new_lens[i])
            width = len(tables[i])
            if cur < 0 or new < cur or -(-new // bs) > width:
                raise AllocError(INVALID, "bad lengths")
            if new > cur and cur % bs != 0:
                b = int(tables[i][cur // bs])
                if not 0 <= b < self.num_blocks:
                    raise AllocError(INVALID, "block id out of range")
                if ref[b] < 1 or (ref[b] > 1 and not cow):
                    raise AllocError(STATE, "appending into a free or shared block")
                if ref[b] > 1:
                    ref[b] -= 1
                    needed += 1
            needed += -(-new // bs) - (-(-cur // bs))
        if needed > self.num_free():
            raise AllocError(OOM, "not enough free blocks")
        slots, copies = [], []
        for i in range(num_seqs):
            row = tables[i]
            cur, new = int(cur_lens[i]), int(new_lens[i])
            if cow and new > cur and cur % bs != 0 and self.ref[int(row[cur // bs])] > 1:
                shared = int(row[cur // bs])
                fresh = self._take()
                self.ref[shared] -= 1
                row[cur // bs] = fresh
                copies.append((shared, fresh))
            for pos in range(cur, new):
                if pos % bs == 0:
                    row[pos // bs] = self._take()
                slots.append(int(row[pos // bs]) * bs + pos % bs)
        return slots, copies

    def trim(self, tables, lens, window: int) -> int:
        """Sliding window: release every block of sequence i that lies wholly
        before its window (16 * (j + 1) <= lens[i] - window) and whose entry
        is not -1; the entry becomes -1. Returns the references released."""
        if window <= 0 or len(tables) != len(lens):
            raise AllocError(INVALID, "bad window or lengths")
        need = {}
        for row, n in zip(tables, lens):
            for j in range(min(max(0, int(n) - window) // self.block_size, len(row))):
                b = int(row[j])
                if b == -1:
                    continue
                if not 0 <= b < self.num_blocks:
                    raise AllocError(INVALID, "block id out of range")
                need[b] = need.get(b, 0) + 1
        for b, c in need.items():
            if self.ref[b] < c:
                raise AllocError(STATE, "releasing a block more times than it is held")
        released = 0
        for row, n in zip(tables, lens):
            for j in range(min(max(0, int(n) - window) // self.block_size, len(row))):
                if int(row[j]) == -1:
                    continue
                self._release(int(row[j]))
                row[j] = -1
                released += 1
        return released

    # -- prefix caching ----------------------------------------------------------
    def register(self, keys, ids) -> int:
        """Name live blocks by content keys; returns how many pairs were taken."""
        ids = [int(b) for b in ids]
        keys = [int(k) for k in keys]
        if len(keys) != len(ids):
            raise AllocError(INVALID, "one key per block")
        self._check_ids(ids)
        for b in ids:
            if self.ref[b] == 0:
                raise AllocError(STATE, "registering a free block")
        taken = 0
        for k, b in zip(keys, ids):
            if b in self.key_of or k in self.block_of:
                continue
            self.key_of[b] = k
            self.block_of[k] = b
            taken += 1
        return taken

    def acquire(self, keys) -> list:
        """Blocks of the longest leading run of known keys, one reference each."""
        out = []
        for k in keys:
            b = self.block_of.get(int(k))
            if b is None:
                break
            if self.ref[b] == 0:
                self.cached.remove(b)
            self.ref[b] += 1
            out.append(b)
        return out
