"""Benchmark of the paged decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload llama13b_layer]
                    [--partition-size PS] [--replicas R] [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch: append each
sequence's new token into its slot (kv_cache_append), decode attention over
the paged cache (paged_attn_decode) and, when partitioned, the split-K merge
(paged_attn_reduce); for a multi-layer workload, all layers. Inputs are
seeded synthetic tensors already resident in HBM. Steps rotate over R
independent replicas of the workload (each with its own pool, tables and
inputs) so that the KV a step reads was not read by the previous R-1 steps:
with R * (pool bytes) well above the 256 MB last-level cache, no step is
served from cache.

Prints one JSON line. `value` is the whole step's KV-read throughput
(algorithmic K+V bytes of the attended tokens / wall time of K back-to-back
steps, synchronized on both sides); a shared prefix counts once per sequence
that attends over it (the effective rate). The roofline counts it once. `roofline` is the decode kernel alone:
the same K launches back to back on the stream they are launched on,
bracketed by one HIP event pair, give its average duration per launch.
`cpu_baseline` is the fp64 oracle on a bounded sample of the same workload.

The 13B-shaped layer runs as a single pass (partition_size 0: every
workgroup covers a whole context, longest sequences first); the long-context
workloads split the context into partitions and merge them with the reduce.
"""

import argparse
import json
import math
import os
import sys
import time

from dataclasses import replace

import numpy as np

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s
BS = 16

# HBM bytes per decode launch from rocprofv3 counter passes: FETCH_SIZE x 2.000
# + WRITE_SIZE x 1.000, the factors read off a copy of known size (1 GiB read
# and written) in the same runs. A figure is reported only while the sources
# of the kernel it was measured on hash to what they were then (their code:
# comments and whitespace are left out of the hash).
_CSRC = "paged_kv_cache_450_amd/csrc/"
KERNEL_SOURCES = {
    "valu": tuple(_CSRC + f for f in ("decode.hip", "decode_core.h", "decode_valu.h", "device.h",
                                       "common.h")),
    "balanced": tuple(_CSRC + f for f in ("decode.hip", "decode_core.h", "decode_valu.h",
                                           "decode_mfma.h", "decode_balanced.h", "device.h",
                                           "common.h")),
    "prefix": tuple(_CSRC + f for f in ("decode.hip", "decode_core.h", "decode_valu.h",
                                         "decode_mfma.h", "decode_balanced.h", "decode_prefix.h",
                                         "device.h", "common.h")),
}
MEASURED_TRAFFIC = {  # traffic_key -> counters of the decode call's streaming kernel
    "llama13b_layer": {  # FETCH 367,277.7 KiB x 1.99992 + WRITE 960.0 KiB
        "kernel": "valu", "bytes": 753_137_682,
        "sources_sha256": "119c792cce40f5982a237eaf91cc3b1b8e22a7fbadf557f3aff8657e5d2a4363",
        "summary": "profiles/decode_kernel_llama13b_layer.md"},
    "longctx_fp8": {  # FETCH 715,843.1 KiB x 1.99998 + WRITE 5,818.3 KiB
        "kernel": "valu", "bytes": 1_471_989_948,
        "sources_sha256": "119c792cce40f5982a237eaf91cc3b1b8e22a7fbadf557f3aff8657e5d2a4363",
        "summary": "profiles/decode_kernel_longctx_fp8.md"},
    "gqa_prefix/shared_prefix_l2": {  # streaming kernel: FETCH 370,925.2 KiB x 1.99995 + WRITE 12,748.9 KiB
        "kernel": "balanced", "bytes": 772_690_692,
        "sources_sha256": "f62bfc6f2a1af97a77860cb808630ee9eb70c636de886a2265a5abc04888ed1d",
        "summary": "profiles/decode_balanced_kernel_gqa_prefix.md"},
    "gqa_prefix/shared_prefix": {  # streaming kernel: FETCH 359,241.7 KiB x 1.99992 + WRITE 12,895.4 KiB
        "kernel": "prefix", "bytes": 748_902_462,
        "sources_sha256": "43a8fd5c11a8653a8e9a8aa76c83349133a9ac87a08a409b583219ec59ba6e0c",
        "summary": "profiles/prefix_kernel_gqa_prefix.md"},
    "7b_32layer": {  # streaming kernel: FETCH 1,049,534.5 KiB x 1.99998 + WRITE 1,536.0 KiB
        "kernel": "balanced", "bytes": 2_150_998_026,
        "sources_sha256": "f62bfc6f2a1af97a77860cb808630ee9eb70c636de886a2265a5abc04888ed1d",
        "summary": "profiles/decode_balanced_kernel_7b_32layer.md"},
}


def _code_only(text: str) -> str:
    """C++ source without its comments, whitespace runs collapsed."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def sources_sha256(kernel: str) -> str:
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(root, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def traffic_key(cfg, w, args=None) -> str:
    """The measured-traffic entry that matches this run: the workload, with
    the options that change what the call launches (args None: the
    workload's default options)."""
    key = cfg.name
    if args is not None and args.unfused:
        key += "/unfused"
    if (args is not None and args.partition_size is not None
            and args.partition_size != cfg.partition_size):
        key += f"/ps{args.partition_size}"
    if w.batch.plan is not None:
        key += "/shared_prefix"
    if w.batch.l2_blocks is not None:
        key += "/shared_prefix_l2"
    if args is not None and args.prefix_tokens:
        key += f"/prompt{args.prefix_tokens}"
    import workloads as W
    base = W.CONFIGS.get(cfg.name, cfg)
    if cfg.q_heads != base.q_heads:
        key += f"/hq{cfg.q_heads}"
    if cfg.balanced != base.balanced:
        key += "/balanced" if cfg.balanced else "/per-sequence"
    return key


def measured_traffic(workload: str):
    entry = MEASURED_TRAFFIC.get(workload)
    if entry is None or entry["sources_sha256"] != sources_sha256(entry["kernel"]):
        return None
    return entry["bytes"]


# ------------------------------------------------------------- workload ----
class Workload:
    """One decode-step workload, product side: pool, tables, inputs, batch."""

    def __init__(self, cfg, seed=0, device="cuda", partition_size=None, fill_byte=None,
                 placement_seed=None, keep_cached_inputs=True, balanced=None, fused=True,
                 shared_prefix=None):
        import torch

        import workloads as W
        from paged_kv_cache_450_amd.runtime import DecodeBatch, PagedKVCache

        self.cfg = cfg
        self.seed = seed
        # fused: a step stores the new tokens inside the decode call
        # (paged_attn_decode_append); else kv_cache_append, then paged_attn_decode.
        self.fused = fused
        lens = W.context_lengths(cfg, seed)
        self.lens = lens
        self.cached = lens - 1
        nb = cfg.pool_blocks or blocks_needed(cfg, lens)
        maxb = -(-int(lens.max()) // BS)
        self.cache = PagedKVCache(cfg.layers, nb, cfg.kv_heads, cfg.head_dim, cfg.kv_dtype,
                                  device, fill_byte=fill_byte)
        pseed = seed if placement_seed is None else placement_seed
        self.cache.permute_free_list(W.free_order(nb, cfg.name, pseed))
        share_from, share_blocks = share_spec(cfg)
        self.tables, self.start, self.slots_cached = self.cache.admit(
            self.cached, maxb, share_from, share_blocks)
        self.slots_new = self.cache.grow(self.tables, self.cached, lens)
        self.partition_size = cfg.partition_size if partition_size is None else partition_size
        qdt = {"f16": torch.float16, "bf16": torch.bfloat16}[cfg.q_dtype]
        self.slots_cached_dev = torch.from_numpy(self.slots_cached).to(device)
        self.slots_new_dev = torch.from_numpy(self.slots_new).to(device)
        self.q, self.k_new, self.v_new = [], [], []
        self.k_cached, self.v_cached = [], []
        self.k_scale, self.v_scale = [], []
        n_cached = int(self.slots_cached.size)
        balanced = cfg.balanced if balanced is None else balanced
        # shared_prefix: the balanced single pass on a 16-bit cache reads the
        # blocks its sequences share once (paged_attn_decode_prefix).
        # (True, or "auto": only when it saves enough repeated reads)
        shared = cfg.shared_prefix if shared_prefix is None else shared_prefix
        if not (balanced and self.partition_size == 0 and cfg.kv_dtype != "e4m3"):
            shared = False
        self.batch = DecodeBatch(self.cache, self.tables, lens, cfg.q_heads, qdt,
                                 self.partition_size, device=device, balanced=balanced,
                                 shared_prefix=shared)
        for layer in range(cfg.layers):
            kc = W.kv_tokens(cfg, seed, layer, "k", "cached", n_cached, device)
            vc = W.kv_tokens(cfg, seed, layer, "v", "cached", n_cached, device)
            kn = W.kv_tokens(cfg, seed, layer, "k", "new", cfg.batch, device)
            vn = W.kv_tokens(cfg, seed, layer, "v", "new", cfg.batch, device)
            ks = vs = None
            if cfg.kv_dtype == "e4m3":
                ks, vs = W.fp8_scales([kc, kn]), W.fp8_scales([vc, vn])
            # prefill: the cached tokens go into their slots
            self.cache.append(layer, kc, vc, self.slots_cached_dev, ks, vs)
            self.q.append(W.q_tensor(cfg, seed, layer, device))
            self.k_new.append(kn)
            self.v_new.append(vn)
            self.k_scale.append(ks)
            self.v_scale.append(vs)
            # keep_cached_inputs: True keeps every layer's prefill rows (the
            # tests compare them), "first" only layer 0's (the CPU baseline).
            if keep_cached_inputs is True or (keep_cached_inputs == "first" and layer == 0):
                self.k_cached.append(kc)
                self.v_cached.append(vc)
            else:
                del kc, vc
        self.out = [None] * cfg.layers

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one decode step reads (attended tokens only),
        counting a shared prefix once per sequence that attends over it."""
        esz = 1 if self.cfg.kv_dtype == "e4m3" else 2
        return int(self.lens.astype(np.int64).sum()) * self.cfg.kv_heads * self.cfg.head_dim * \
            2 * esz * self.cfg.layers

    def kv_unique_bytes(self) -> int:
        """The same, counting each shared prefix block once: the bytes that
        must come from HBM."""
        import workloads as W
        esz = 1 if self.cfg.kv_dtype == "e4m3" else 2
        tokens = int(self.lens.astype(np.int64).sum())
        sh = W.sharers(self.cfg)
        if len(sh) > 1:
            tokens -= (len(sh) - 1) * self.cfg.share_prefix_tokens
        return tokens * self.cfg.kv_heads * self.cfg.head_dim * 2 * esz * self.cfg.layers

    def append(self, layer, stream=None):
        self.cache.append(layer, self.k_new[layer], self.v_new[layer], self.slots_new_dev,
                          self.k_scale[layer], self.v_scale[layer], stream)

    def decode(self, layer, stream=None):
        self.batch.k_scale, self.batch.v_scale = self.k_scale[layer], self.v_scale[layer]
        self.batch.decode(layer, self.q[layer], stream)

    def reduce(self, stream=None):
        self.batch.reduce(stream)

    def decode_append(self, layer, stream=None):
        self.batch.k_scale, self.batch.v_scale = self.k_scale[layer], self.v_scale[layer]
        self.batch.decode_append(layer, self.q[layer], self.k_new[layer], self.v_new[layer],
                                 stream)

    def step(self, layer=None, stream=None):
        layers = range(self.cfg.layers) if layer is None else [layer]
        for l in layers:
            if self.fused:
                self.decode_append(l, stream)
            else:
                self.append(l, stream)
                self.decode(l, stream)
            self.reduce(stream)
        return self.batch.out


def decode_kernel_name(cfg, w) -> str:
    """The kernel(s) one paged_attn_decode call of this workload runs."""
    grouped = cfg.q_heads > cfg.kv_heads and cfg.kv_dtype != "e4m3"
    if w.partition_size == 0 and w.batch.balanced:
        if w.batch.plan is not None and w.batch.plan.num_groups > 0:
            return "prefix_kernel + decode_balanced_kernel + balanced_merge_kernel"
        return "decode_balanced_kernel + balanced_merge_kernel"
    return "decode_mfma_kernel" if grouped else "decode_kernel"


def blocks_needed(cfg, lens) -> int:
    import workloads as W
    n = int(sum(-(-int(l) // BS) for l in lens))
    sh = W.sharers(cfg)
    if len(sh) > 1:
        n -= (len(sh) - 1) * (cfg.share_prefix_tokens // BS)
    return n


def share_spec(cfg):
    import workloads as W
    sh = W.sharers(cfg)
    share_from = np.full(cfg.batch, -1, dtype=np.int64)
    for i in sh[1:]:
        share_from[i] = sh[0]
    return share_from, cfg.share_prefix_tokens // BS


# ------------------------------------------------------------ oracle side ----
class OracleBookkeeping:
    """The same admission procedure run on the oracle's AllocatorModel (used by
    the CPU baseline and by the tests; never by the timed GPU path)."""

    def __init__(self, cfg, seed=0, placement_seed=None):
        from oracle import allocator as oalloc
        import workloads as W

        lens = W.context_lengths(cfg, seed)
        cached = lens - 1
        nb = cfg.pool_blocks or blocks_needed(cfg, lens)
        maxb = -(-int(lens.max()) // BS)
        model = oalloc.AllocatorModel(nb, BS)
        model.alloc(nb)
        pseed = seed if placement_seed is None else placement_seed
        model.free([int(x) for x in W.free_order(nb, cfg.name, pseed)])
        share_from, share_blocks = share_spec(cfg)
        rows = [[-1] * maxb for _ in range(cfg.batch)]
        start = np.zeros(cfg.batch, dtype=np.int32)
        slots = []
        for i in range(cfg.batch):
            if share_from[i] >= 0:
                model.fork(rows[share_from[i]], rows[i], share_blocks)
                start[i] = share_blocks * BS
            slots += model.extend([rows[i]], [int(start[i])], [int(cached[i])])
        slots_new = model.extend(rows, [int(c) for c in cached], [int(x) for x in lens])
        self.model = model
        self.lens = lens
        self.tables = np.array(rows, dtype=np.int32)
        self.start = start
        self.slots_cached = np.array(slots, dtype=np.int64)
        self.slots_new = np.array(slots_new, dtype=np.int64)

    def token_offsets(self):
        """offs[i]:offs[i+1] index the cached-token inputs written for sequence i."""
        counts = (self.lens.astype(np.int64) - 1 - self.start)
        return np.concatenate([[0], np.cumsum(counts)])


def _oracle_worker(job):
    """One worker of cpu_baseline's parallel leg, in a spawned process of its
    own (one BLAS thread): maps the oracle's host pool read-only from a file
    and runs the oracle's decode over its share of the sequences, whole passes
    until its budget is spent. Returns its start and end on the system-wide
    monotonic clock, the KV bytes it decoded and the sequences it did."""
    from oracle import attention as oattn

    path, shape, dtype, rows, lens, qs, scale, kv_dtype, ks, vs, esz, budget = job
    p6 = np.memmap(path, dtype=dtype, mode="r", shape=shape)
    t_start = time.monotonic()
    elapsed, done, seqs = 0.0, 0, 0
    while elapsed < budget:
        for row, n, q in zip(rows, lens, qs):
            t0 = time.perf_counter()
            oattn.paged_decode(p6, 0, q, row[None], np.array([n]), scale, kv_dtype, ks, vs)
            elapsed += time.perf_counter() - t0
            done += int(n) * shape[3] * shape[5] * 2 * esz
            seqs += 1
            if elapsed >= budget:
                break
    t_end = time.monotonic()
    del p6
    return t_start, t_end, done, seqs


def cpu_baseline(w: Workload, budget_s: float, workers=None):
    """The fp64 oracle, as it is, on a bounded sample of the same workload:
    whole sequences, in order, until about budget_s of CPU work. Only the
    oracle's decode (gather through the table, softmax, PV) is timed; its
    host pool is built by the oracle's own append, with the oracle's own
    bookkeeping, from host copies of the seeded inputs.

    Two legs: `value` runs the sequences over `workers` spawned processes at
    once (one BLAS thread each; the oracle's per-head loop uses one core per
    process), as many as the host's cores allow up to 16, and reports the
    aggregate rate over the wall time from the first worker's start to the
    last one's end; `single_thread` runs them in this process with BLAS
    limited to one thread."""
    import multiprocessing as mp
    import tempfile

    import torch

    from oracle import attention as oattn
    from oracle import pool as opool

    cfg = w.cfg
    ob = OracleBookkeeping(cfg, w.seed)
    offs = ob.token_offsets()

    def raw(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    nb = ob.model.num_blocks
    per_layer = opool.pool_bytes(1, nb, BS, cfg.kv_heads, cfg.head_dim, cfg.kv_dtype)
    shm_dir = "/dev/shm" if os.path.isdir("/dev/shm") else None
    tmp = tempfile.NamedTemporaryFile(prefix="pkv_oracle_pool_", dir=shm_dir, delete=False)
    tmp.close()
    try:
        buf = np.memmap(tmp.name, dtype=np.uint8, mode="w+", shape=(per_layer,))
        p6 = opool.view_pool(buf, 1, nb, BS, cfg.kv_heads, cfg.head_dim, cfg.kv_dtype)
        ks = vs = None
        if cfg.kv_dtype == "e4m3":
            ks, vs = w.k_scale[0].cpu().numpy(), w.v_scale[0].cpu().numpy()
        scale = float(np.float32(1.0 / math.sqrt(cfg.head_dim)))
        esz = opool.ESIZE[cfg.kv_dtype]
        # Host pool: the oracle's own append of every private sequence's tokens.
        todo = []
        for i in range(cfg.batch):
            if ob.start[i] > 0:
                continue  # a prefix sharer; its prefix owner's tokens are not in this host pool
            lo, hi = int(offs[i]), int(offs[i + 1])
            opool.append(p6, 0, raw(w.k_cached[0][lo:hi]), raw(w.v_cached[0][lo:hi]),
                         cfg.src_dtype, cfg.kv_dtype, ob.slots_cached[lo:hi], ks, vs)
            opool.append(p6, 0, raw(w.k_new[0][i:i + 1]), raw(w.v_new[0][i:i + 1]), cfg.src_dtype,
                         cfg.kv_dtype, ob.slots_new[i:i + 1], ks, vs)
            todo.append((i, opool.raw_to_f64(raw(w.q[0][i:i + 1]), cfg.q_dtype)))
        buf.flush()

        def what(seqs, passes, done, secs):
            return (f"{seqs} sequence decodes ({passes} over the {len(todo)} sequences of "
                    f"{cfg.name} layer 0; {done / 1e6:.1f} MB of KV), fp64 numpy decode only, "
                    f"{secs:.1f} s")

        # Parallel leg: sequences dealt round robin to the workers.
        n_work = workers or max(1, min(16, os.cpu_count() or 1, len(todo)))
        jobs = []
        for k in range(n_work):
            mine = todo[k::n_work]
            jobs.append((tmp.name, p6.shape, p6.dtype, [ob.tables[i] for i, _ in mine],
                         [int(ob.lens[i]) for i, _ in mine], [q for _, q in mine], scale,
                         cfg.kv_dtype, ks, vs, esz, budget_s))
        saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                                 "MKL_NUM_THREADS")}
        os.environ.update({k: "1" for k in saved})
        try:
            with mp.get_context("spawn").Pool(n_work) as pool:
                res = pool.map(_oracle_worker, jobs, chunksize=1)
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
        wall = max(r[1] for r in res) - min(r[0] for r in res)
        done = sum(r[2] for r in res)
        seqs = sum(r[3] for r in res)
        par = {"value": round(done / wall / 1e9, 4), "seqs_per_s": round(seqs / wall, 3),
               "sample": what(seqs, "whole passes of each worker", done, wall)
               + f" of wall time on {n_work} worker processes"}

        def run(budget):
            """Whole passes over those sequences until about budget s of oracle decode."""
            elapsed, done_bytes, nseq, passes = 0.0, 0, 0, 0
            while elapsed < budget and todo:
                for i, q in todo:
                    t0 = time.perf_counter()
                    oattn.paged_decode(p6, 0, q, ob.tables[i:i + 1], ob.lens[i:i + 1], scale,
                                       cfg.kv_dtype, ks, vs)
                    elapsed += time.perf_counter() - t0
                    done_bytes += int(ob.lens[i]) * cfg.kv_heads * cfg.head_dim * 2 * esz
                    nseq += 1
                    if elapsed >= budget:
                        break
                passes += 1
            return {"value": round(done_bytes / elapsed / 1e9, 4),
                    "seqs_per_s": round(nseq / elapsed, 3),
                    "sample": what(nseq, f"{passes} passes", done_bytes, elapsed)}

        single = None
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                single = run(budget_s / 2)
        except ImportError:
            pass
        del p6, buf
    finally:
        os.unlink(tmp.name)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                         "")
    except OSError:
        pass
    out = {"value": par["value"], "unit": "GB/s", "cores": n_work, "kind": "oracle",
           "sample": par["sample"], "seqs_per_s": par["seqs_per_s"],
           "cpu_count": os.cpu_count(), "cpu_model": model}
    if single is not None:
        out["single_thread"] = {"value": single["value"], "unit": "GB/s", "cores": 1,
                                "seqs_per_s": single["seqs_per_s"], "sample": single["sample"]}
    return out


def block_copy_rate(cfg, pairs: int, iters: int, stream) -> dict:
    """kv_block_copy of `pairs` blocks (every layer, K and V) into fresh blocks
    of a pool of the workload's geometry, timed over `iters` calls back to back
    with one event pair; bytes = read + written."""
    import torch

    import paged_kv_cache_450_amd as P
    from paged_kv_cache_450_amd.runtime import PagedKVCache

    cache = PagedKVCache(cfg.layers, 2 * pairs, cfg.kv_heads, cfg.head_dim, cfg.kv_dtype, "cuda",
                         fill_byte=1)
    rng = np.random.default_rng(0)
    src = rng.permutation(pairs).astype(np.int32)
    dst = (pairs + rng.permutation(pairs)).astype(np.int32)
    P.kv_block_copy(cache.handle, src, dst, stream)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(iters):
        P.kv_block_copy(cache.handle, src, dst, stream)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / iters * 1e3
    esz = 1 if cfg.kv_dtype == "e4m3" else 2
    block_bytes = cfg.layers * 2 * cfg.kv_heads * BS * cfg.head_dim * esz
    moved = 2 * pairs * block_bytes
    cache.close()
    return {"pairs": pairs, "bytes_per_block": block_bytes, "us": round(us, 3),
            "GBs": round(moved / (us * 1e-6) / 1e9, 1),
            "frac_hbm": round(moved / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def swap_rate(cfg, blocks: int, iters: int, stream) -> dict:
    """kv_swap_out of `blocks` random blocks (every layer, K and V) of a pool of
    the workload's geometry into pinned host slots, and kv_swap_in back, each
    timed over `iters` calls back to back with one event pair; bytes = one
    slot per block each way. For reference, the copy engine's rate on a
    contiguous device <-> pinned host copy of the same size."""
    import torch

    import paged_kv_cache_450_amd as P
    from paged_kv_cache_450_amd.runtime import PagedKVCache

    cache = PagedKVCache(cfg.layers, 2 * blocks, cfg.kv_heads, cfg.head_dim, cfg.kv_dtype,
                         "cuda", fill_byte=1)
    h = cache.handle
    slot = P.kv_swap_slot_bytes(h)
    host = torch.empty(blocks * slot, dtype=torch.uint8, pin_memory=True)
    rng = np.random.default_rng(0)
    ids = rng.permutation(2 * blocks)[:blocks].astype(np.int32)
    slots = rng.permutation(blocks).astype(np.int32)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(iters):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / iters * 1e3

    out_us = timed(lambda: P.kv_swap_out(h, ids, slots, host, stream))
    in_us = timed(lambda: P.kv_swap_in(h, slots, ids, host, stream))
    dev = torch.empty(blocks * slot, dtype=torch.uint8, device="cuda")
    with torch.cuda.stream(stream):
        d2h_us = timed(lambda: host.copy_(dev, non_blocking=True))
        h2d_us = timed(lambda: dev.copy_(host, non_blocking=True))
    moved = blocks * slot
    cache.close()

    def gbs(us):
        return round(moved / (us * 1e-6) / 1e9, 2)
    return {"blocks": blocks, "bytes_per_block": slot, "out_us": round(out_us, 2),
            "out_GBs": gbs(out_us), "in_us": round(in_us, 2), "in_GBs": gbs(in_us),
            "copy_engine_d2h_GBs": gbs(d2h_us), "copy_engine_h2d_GBs": gbs(h2d_us)}


def serving_rate(cfg, iters: int, stream, groups=(0, 0), caching=False, swap_slots=0,
                 pool_blocks=0, max_gen=128, window=0, shared_prefix=False) -> dict:
    """The continuous-batching loop (ContinuousBatcher) over a seeded request
    stream shaped like the workload: prompts of up to its longest context, 1 to
    max_gen generated tokens, a third of the requests with 2-3 samples, 4 arrivals
    per iteration and a pool of the workload's size (so requests queue and, at
    times, are preempted). groups = (G, T): prompts in G prefix groups sharing
    their first T tokens (a system prompt); caching: admit through the prefix
    cache; swap_slots: preempt into a swap space of that many pinned host slots
    (else by recomputation); window > 0: a sliding window of that many tokens
    (blocks before it released every iteration); pool_blocks > 0: a pool of that many blocks
    instead (a tight pool forces preemption); shared_prefix (True or "auto"): the balanced
    pass with the shared-prefix pass, planned every iteration. Inputs are drawn before the
    timed region, which holds the bookkeeping (host) and the GPU work of every iteration."""
    import torch

    import workloads as W
    from paged_kv_cache_450_amd.runtime import ContinuousBatcher, PagedKVCache, SwapSpace

    lens = W.context_lengths(cfg, 0)
    max_prompt = int(lens.max())
    max_prompt = max(max_prompt, groups[1])
    nb = pool_blocks or cfg.pool_blocks or blocks_needed(cfg, lens)
    width = -(-(max_prompt + max_gen) // BS)
    trace = W.request_trace(cfg.name + "_serve", 0, 4 * iters, max_prompt, max_gen,
                            mean_gap=0.25, prefix_groups=groups[0], shared_tokens=groups[1])
    cache = PagedKVCache(cfg.layers, nb, cfg.kv_heads, cfg.head_dim, cfg.kv_dtype, "cuda")
    swap = SwapSpace(cache, swap_slots) if swap_slots else None
    loop = ContinuousBatcher(cache, width, prefix_caching=caching, swap=swap, window=window)
    dt = cfg.src_dtype
    kp = W.normal((max_prompt, cfg.kv_heads, cfg.head_dim), dt, 1, "cuda")
    vp = W.normal((max_prompt, cfg.kv_heads, cfg.head_dim), dt, 2, "cuda")
    cap = 4096
    qs = W.normal((cap, cfg.q_heads, cfg.head_dim), cfg.q_dtype, 3, "cuda")
    ks = W.normal((cap, cfg.kv_heads, cfg.head_dim), dt, 4, "cuda")
    vs = W.normal((cap, cfg.kv_heads, cfg.head_dim), dt, 5, "cuda")
    k_scale = v_scale = None
    if cfg.kv_dtype == "e4m3":
        k_scale, v_scale = W.fp8_scales([kp, ks]), W.fp8_scales([vp, vs])
    # the workload's single-pass form: balanced (with a workspace) or per sequence;
    # the shared-prefix pass needs the balanced one and a workspace for the batch
    if shared_prefix:
        import paged_kv_cache_450_amd as P
        wsb = P.paged_attn_prefix_workspace_bytes(cap, cfg.q_heads, cfg.head_dim)
    else:
        wsb = P_workspace_bytes(cfg) if cfg.balanced else 0
    workspace = torch.empty(wsb // 4, dtype=torch.float32, device="cuda") if wsb else None

    def prompt_kv(spec, layer):
        return kp[:spec.prompt_len], vp[:spec.prompt_len]

    def step_inputs(layer, n):
        return qs[:n], ks[:n], vs[:n]

    pending = list(trace)
    host_s = 0.0
    tokens = copies = preempted = prefill = reused = swapped_out = swapped_blocks = done = 0
    discarded = 0  # tokens generated by requests that recomputation then restarted
    released = 0   # block references released by the window
    batches = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for it in range(iters):
        while pending and pending[0].arrival <= it:
            loop.submit(pending.pop(0))
        gen = {}
        for sq in loop.running:
            gen[sq.rid] = gen.get(sq.rid, 0) + sq.generated
        h0 = time.perf_counter()
        plan = loop.plan()
        host_s += time.perf_counter() - h0
        loop.execute(plan, prompt_kv, step_inputs, cfg.q_heads, k_scale=k_scale,
                     v_scale=v_scale, workspace=workspace, stream=stream,
                     shared_prefix=shared_prefix)
        tokens += len(plan.batch)
        prefill += sum(int(a[2].size) for a in plan.admitted)
        reused += sum(a[1] // BS for a in plan.admitted)
        batches.append(len(plan.batch))
        copies += len(plan.copy_src) if plan.copy_src is not None else 0
        preempted += len(plan.preempted)
        discarded += sum(gen.get(r, 0) for r in plan.preempted)
        swapped_out += len(plan.swapped_out)
        done += len(plan.finished)
        released += plan.trimmed
        swapped_blocks += len(plan.swap_out_ids) + len(plan.swap_in_ids)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cache.close()
    return {"iterations": iters, "decode_tokens": tokens, "tokens_per_s": round(tokens / wall, 1),
            "sequences_finished": done, "sequences_finished_per_s": round(done / wall, 1),
            "ms_per_iteration": round(wall / iters * 1e3, 4),
            "host_plan_us_per_iteration": round(host_s / iters * 1e6, 1),
            "mean_batch": round(float(np.mean(batches)), 2), "max_batch": int(max(batches)),
            "copies": copies, "preemptions": preempted, "tokens_discarded": discarded,
            "max_gen": max_gen, "swap_slots": swap_slots, "window": window,
            "blocks_released_by_window": released,
            "swapped_out": swapped_out, "blocks_swapped": swapped_blocks, "pool_blocks": nb,
            "prefix_caching": caching, "prefix_groups": list(groups),
            "shared_prefix": shared_prefix, "shared_prefix_groups_run": loop.prefix_groups_run,
            "prefill_tokens": prefill, "cached_blocks_reused": reused,
            "requests_admitted": 4 * iters - len(pending) - len(loop.waiting)}


def window_rate(ws, window: int, steps: int, stream, fused: bool, full_us: float) -> dict:
    """The step with a sliding window of `window` tokens on the same caches:
    per layer, the decode call (storing the new tokens when fused) and the
    reduce, timed back to back over the replicas like the full-context step.
    Bytes are those of the attended tokens, min(L, window) per sequence."""
    import torch

    cfg = ws[0].cfg
    esz = 1 if cfg.kv_dtype == "e4m3" else 2
    per_token = cfg.kv_heads * cfg.head_dim * 2 * esz
    attended = [int(np.minimum(w.lens, window).astype(np.int64).sum()) * per_token for w in ws]
    for w in ws:
        w.batch.window = window
    try:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(len(ws)):  # warm-up
            ws[i].step(stream=stream)
        torch.cuda.synchronize()
        a.record(stream)
        n = 0
        for i in range(steps):
            w = ws[i % len(ws)]
            for layer in range(cfg.layers):
                if fused:
                    w.decode_append(layer, stream)
                else:
                    w.decode(layer, stream)
                w.reduce(stream)
                n += 1
        b.record(stream)
        torch.cuda.synchronize()
    finally:
        for w in ws:
            w.batch.window = 0
    us = a.elapsed_time(b) / n * 1e3
    per_call = sum(attended) / len(attended)
    return {"window": window, "attended_bytes_per_layer": int(per_call),
            "us_per_layer": round(us, 3), "GB/s": round(per_call / (us * 1e-6) / 1e9, 2),
            "seqs_per_s_per_layer": round(cfg.batch / (us * 1e-6), 1),
            "full_context_us_per_layer": round(full_us, 3)}


# The other workloads the default run reports beside the 13B layer:
# (name, warm-up steps, timed steps).
OTHER_CONFIGS = (("tiny", 20, 200), ("7b_32layer", 2, 5), ("gqa_prefix", 10, 100),
                 ("longctx_fp8", 10, 50))


def config_summary(name: str, seed: int, warmup: int, steps: int, stream) -> dict:
    """One workload in its default form, measured as the main line measures
    the 13B layer: `steps` whole steps back to back over replicas of >= 2 GB in
    total (wall clock, synchronized on both sides), then the decode call alone
    (per layer, as the step makes it; the split-K reduce separately), each
    launched `steps` x layers times back to back between one HIP event pair.
    The roofline figure is the decode call's unique KV bytes over its time."""
    import torch

    import workloads as W

    cfg = W.CONFIGS[name]
    t_build = time.perf_counter()
    first = Workload(cfg, seed, "cuda", keep_cached_inputs=False)
    reps = max(1, min(8, math.ceil(2e9 / max(first.cache.nbytes, 1))))
    ws = [first] + [Workload(cfg, seed + r, "cuda", keep_cached_inputs=False)
                    for r in range(1, reps)]
    t_build = time.perf_counter() - t_build
    kv = sum(w.kv_bytes() for w in ws) / reps
    uniq = sum(w.kv_unique_bytes() for w in ws) / reps
    nl = cfg.layers
    for i in range(warmup):
        ws[i % reps].step(stream=stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ws[i % reps].step(stream=stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps

    def per_launch_us(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(steps):
            for layer in range(nl):
                fn(ws[i % reps], layer)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (steps * nl) * 1e3

    decode_us = per_launch_us(lambda w, l: w.decode_append(l, stream))
    reduce_us = (per_launch_us(lambda w, l: w.reduce(stream)) if first.partition_size > 0
                 else 0.0)
    per_layer_unique = uniq / nl
    rate = per_layer_unique / (decode_us * 1e-6) / 1e9
    out = {
        "layers": nl, "batch": cfg.batch, "q_heads": cfg.q_heads, "kv_heads": cfg.kv_heads,
        "head_dim": cfg.head_dim, "kv_dtype": cfg.kv_dtype, "context_lens": list(cfg.lengths),
        "partition_size": first.partition_size,
        "single_pass": ("balanced" if first.batch.balanced else "per-sequence")
        if first.partition_size == 0 else None,
        "replicas": reps, "steps": steps, "warmup": warmup,
        "ms_per_step": round(wall * 1e3, 5),
        "GB/s": round(kv / wall / 1e9, 2), "pct_hbm_peak": round(100 * kv / wall / 1e9 /
                                                                 HBM_PEAK_GBS, 2),
        "seqs_per_s": round(cfg.batch / wall, 1),
        "kv_bytes_per_step": int(kv), "kv_unique_bytes_per_step": int(uniq),
        "decode_call_us_per_layer": round(decode_us, 3), "reduce_us": round(reduce_us, 3),
        "roofline": {"bound": "hbm", "kernel": decode_kernel_name(cfg, first),
                     "achieved": round(rate, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(rate / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(traffic_key(cfg, first)),
                     "algorithmic_bytes": int(per_layer_unique)},
        "setup_s": round(t_build, 1),
    }
    if cfg.batch <= 8 and kv < 1e7:
        out["latency_us_per_step"] = round(wall * 1e6, 2)
    for w in ws:
        w.cache.close()
    del ws, first
    # The freed device memory stays in torch's cache for the next workload:
    # handed back to the driver, it would be reclaimed in the background while
    # the next workload is timed (about 35 s per 100 GB, costing a
    # bandwidth-bound kernel about 3%: the GQA call 142.6 against 139.6-140.0 us
    # after the 7B pools).
    torch.cuda.synchronize()
    return out


def gather_probe(stream, iters: int = 20) -> dict:
    """The decode's memory access pattern alone (libpkvprobe.so): waves
    streaming random 4 KiB K tiles and the matching V tiles from two 1 GiB
    planes, 16-byte non-temporal loads, no arithmetic. The rate the
    scattered tiles reach is the decode kernels' practical ceiling on this
    GPU. Staged through a ring of three tiles in registers (the decode's form)
    or a ring of two or three tiles in LDS filled by direct buffer-to-LDS
    loads, at several waves per workgroup; each form launched `iters` times
    back to back between one HIP event pair. Two sizes: 5120 waves x 51 tiles
    (2.14 GB per launch) and 5120 x 18 (755 MB, the 13B layer's size)."""
    import ctypes

    import torch

    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "paged_kv_cache_450_amd",
                        "libpkvprobe.so")
    lib = ctypes.CDLL(path)
    fn = lib.pkv_probe_gather
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    fn.restype = ctypes.c_int
    fn.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]
    num_tiles = 1 << 18  # 1 GiB per plane
    kp = torch.full((num_tiles * 4096,), 1, dtype=torch.uint8, device="cuda")
    vpl = torch.full((num_tiles * 4096,), 2, dtype=torch.uint8, device="cuda")
    num_waves = 5120
    rng = np.random.default_rng(0)
    perm = rng.permutation(num_tiles).astype(np.int32)

    def run_ids(run: int, per_wave: int) -> np.ndarray:
        """Tile k of consecutive waves 0..run-1 of each group of `run` waves
        are `run` adjacent tiles (a block's adjacent kv heads in the pool):
        the group's concurrent loads form one run of run x 4 KiB."""
        groups = num_waves // run
        starts = rng.permutation(num_tiles // run)[: groups * per_wave].astype(np.int64) * run
        ids = starts.reshape(groups, per_wave)[:, None, :] + np.arange(run)[None, :, None]
        return ids.reshape(num_waves, per_wave).astype(np.int32)

    layouts = {"random": perm[: num_waves * 51].copy(), "runs of 4": run_ids(4, 51).ravel(),
               "runs of 40": run_ids(40, 51).ravel()}
    sink = torch.zeros(num_waves * 64, dtype=torch.int32, device="cuda")
    st = stream.cuda_stream
    out = []
    for layout, per_wave, forms in (
            ("random", 51, ((0, 4), (0, 1), (1, 1), (1, 2), (1, 4), (2, 1), (2, 2))),
            ("random", 18, ((0, 4), (1, 1), (1, 4), (2, 1))),
            ("runs of 4", 51, ((0, 4), (1, 4))), ("runs of 40", 51, ((0, 4), (1, 4)))):
        host = layouts[layout]
        if per_wave != 51:
            host = host[: num_waves * per_wave]
        ids = torch.from_numpy(np.ascontiguousarray(host)).cuda()
        for mode, wpg in forms:
            def launch():
                rc = fn(kp.data_ptr(), vpl.data_ptr(), ids.data_ptr(), num_waves, per_wave,
                        num_tiles, mode, wpg, sink.data_ptr(), st)
                if rc != 0:
                    raise RuntimeError(f"pkv_probe_gather: hip error {rc}")
            for _ in range(3):
                launch()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(iters):
                launch()
            b.record(stream)
            torch.cuda.synchronize()
            us = a.elapsed_time(b) / iters * 1e3
            nbytes = num_waves * per_wave * 8192
            out.append({"staging": ["registers, 3 tiles", "LDS, 2 tiles", "LDS, 3 tiles"][mode],
                        "tile_layout": layout,
                        "waves_per_workgroup": wpg, "tiles_per_wave": per_wave,
                        "bytes_per_launch": nbytes, "us": round(us, 2),
                        "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1)})
    del kp, vpl, ids, sink
    torch.cuda.empty_cache()
    return {"forms": out}


def P_workspace_bytes(cfg) -> int:
    import paged_kv_cache_450_amd as P
    return P.paged_attn_workspace_bytes(1, cfg.q_heads, cfg.head_dim, 1, 0)


# --shared-prefix choices -> DecodeBatch(shared_prefix=...)
SHARED_FORMS = {None: None, "kernel": True, "l2": "l2", "auto": "auto"}


# ------------------------------------------------------------------ main ----
def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama13b_layer")
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--replicas", type=int, default=None,
                    help="independent copies rotated over (default: enough for >= 2 GB)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--block-copy", type=int, default=0, metavar="N",
                    help="also time kv_block_copy of N block pairs (copy on write) on a pool of "
                         "the workload's geometry")
    ap.add_argument("--serve", type=int, default=0, metavar="ITERS",
                    help="also run the continuous-batching loop for ITERS iterations on a "
                         "request stream of the workload's shape and report its rates")
    ap.add_argument("--serve-prefix", default=None, metavar="GROUPS,TOKENS",
                    help="serving stream with prompts in GROUPS prefix groups sharing their "
                         "first TOKENS tokens")
    ap.add_argument("--serve-caching", action="store_true",
                    help="run the serving loop with prefix caching")
    ap.add_argument("--swap", type=int, default=0, metavar="N",
                    help="also time kv_swap_out / kv_swap_in of N blocks of the workload's "
                         "geometry to and from pinned host memory")
    ap.add_argument("--serve-swap", type=int, default=0, metavar="SLOTS",
                    help="run the serving loop with a swap space of SLOTS host slots")
    ap.add_argument("--serve-blocks", type=int, default=0, metavar="N",
                    help="run the serving loop on a pool of N blocks")
    ap.add_argument("--serve-gen", type=int, default=128, metavar="N",
                    help="longest generation of the serving stream's requests")
    ap.add_argument("--serve-shared-prefix", choices=["on", "auto"], default=None,
                    help="run the serving loop's decode with the shared-prefix pass (always, "
                         "or when it saves enough repeated reads)")
    ap.add_argument("--serve-window", type=int, default=0, metavar="W",
                    help="run the serving loop with a sliding window of W tokens")
    ap.add_argument("--window", default=None, metavar="W[,W...]",
                    help="also time the step with a sliding window of W tokens "
                         "(paged_attn_decode_window) on the same caches")
    ap.add_argument("--unfused", action="store_true",
                    help="run a step as kv_cache_append + paged_attn_decode instead of the "
                         "fused paged_attn_decode_append")
    ap.add_argument("--prefix-tokens", type=int, default=0, metavar="N",
                    help="lengthen the shared prompt of a workload with one (gqa_prefix) to N "
                         "tokens; its sharers' contexts grow to at least N + 1")
    ap.add_argument("--shared-prefix", nargs="?", const="kernel", default=None,
                    choices=["kernel", "l2", "auto"],
                    help="read blocks that several sequences share once per step with the prefix "
                         "kernel (paged_attn_decode_prefix; the default when given alone), or "
                         "through the L2 in the balanced pass (l2: paged_attn_decode_prefix_l2)")
    ap.add_argument("--q-heads", type=int, default=0, metavar="HQ",
                    help="run the workload with HQ query heads (a multiple of its kv heads) on "
                         "the same pool, tables and lengths: another head grouping of the same "
                         "KV bytes")
    ap.add_argument("--single-pass", choices=["balanced", "per-sequence"], default=None,
                    help="the single-pass form instead of the workload's own")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gather-probe", action="store_true",
                    help="also measure the rate of the decode's access pattern alone (random "
                         "4 KiB K and V tiles) with register and LDS staging")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the other workloads the default 13B run also reports")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain elementwise copy of this many MiB before warm-up: a "
                         "kernel of known traffic against which profiler byte counters are "
                         "calibrated")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the paged decode path has no multi-GPU "
              "component here (run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    cfg = W.CONFIGS[args.workload]
    if args.prefix_tokens > 0:
        if not cfg.share_prefix_tokens:
            print(f"--prefix-tokens: workload {cfg.name} has no shared prompt", file=sys.stderr)
            return 2
        cfg = replace(cfg, share_prefix_tokens=args.prefix_tokens)
    if args.q_heads:
        if args.q_heads % cfg.kv_heads or args.q_heads // cfg.kv_heads not in (1, 2, 4, 8):
            print(f"--q-heads: {args.q_heads} query heads for {cfg.kv_heads} kv heads",
                  file=sys.stderr)
            return 2
        cfg = replace(cfg, q_heads=args.q_heads)
    if args.single_pass is not None:
        cfg = replace(cfg, balanced=args.single_pass == "balanced")
    torch.cuda.set_device(0)
    fused = not args.unfused
    first = Workload(cfg, args.seed, "cuda", args.partition_size,
                     keep_cached_inputs=False if args.no_cpu_baseline else "first", fused=fused,
                     shared_prefix=SHARED_FORMS[args.shared_prefix])
    pool_bytes = first.cache.nbytes
    reps = args.replicas or max(1, min(8, math.ceil(2e9 / max(pool_bytes, 1))))
    ws = [first] + [Workload(cfg, args.seed + r, "cuda", args.partition_size,
                             keep_cached_inputs=False, fused=fused,
                             shared_prefix=SHARED_FORMS[args.shared_prefix])
                    for r in range(1, reps)]
    kv_bytes = [w.kv_bytes() for w in ws]
    kv_unique = [w.kv_unique_bytes() for w in ws]
    stream = torch.cuda.current_stream()
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 18  # fp32 elements
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)  # reads and writes exactly 4n bytes each
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()

    for i in range(args.warmup):
        ws[i % reps].step(stream=stream)
    torch.cuda.synchronize()

    # Timed region: exactly K whole steps back to back, synchronized on both
    # sides; one event pair on the launch stream brackets the region (an event
    # record between kernels costs a few microseconds of GPU time, so none is
    # placed inside a step).
    nl = cfg.layers
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    bytes_done = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        bytes_done += kv_bytes[i % reps]
        ws[i % reps].step(stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) / args.steps * 1e3
    gpu_ms_per_step = e0.elapsed_time(e1) / args.steps
    gbs = bytes_done / (t1 - t0) / 1e9

    # Per-kernel durations: each kernel launched K*layers times back to back on
    # the same stream (same replica rotation and arguments as the steps),
    # bracketed by one event pair; average duration per launch.
    def per_launch_us(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(args.steps):
            for layer in range(nl):
                fn(ws[i % reps], layer)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (args.steps * nl) * 1e3

    # The decode call as the step makes it (fused: it also stores the new
    # tokens), and the separate append kernel for reference.
    if fused:
        decode_us = per_launch_us(lambda w, l: w.decode_append(l, stream))
    else:
        decode_us = per_launch_us(lambda w, l: w.decode(l, stream))
    append_us = per_launch_us(lambda w, l: w.append(l, stream))
    reduce_us = (per_launch_us(lambda w, l: w.reduce(stream))
                 if first.partition_size > 0 else 0.0)
    # Distribution of the decode call's duration: one event pair around each of
    # K launches (outside the timed region; each pair adds a little GPU time).
    call_us = []
    for i in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w = ws[i % reps]
        a.record(stream)
        if fused:
            w.decode_append(i % nl, stream)
        else:
            w.decode(i % nl, stream)
        b.record(stream)
        call_us.append((a, b))
    torch.cuda.synchronize()
    call_us = np.array([a.elapsed_time(b) * 1e3 for a, b in call_us])
    per_layer_bytes = sum(kv_bytes) / reps / nl
    # The roofline counts the bytes that must come from HBM: a shared prefix once.
    per_layer_unique = sum(kv_unique) / reps / nl
    decode_gbs = per_layer_unique / (decode_us * 1e-6) / 1e9

    result = {
        "metric": "paged decode-attn KV-read GB/s (% HBM peak) + seqs/s at 13B shape, 1 GPU",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.kv_dtype,
        "data": "synthetic",
        "config": {
            "workload": cfg.name,
            "single_pass": ("balanced" if first.batch.balanced else "per-sequence")
            if first.partition_size == 0 else None,
            "layers": cfg.layers, "batch": cfg.batch, "q_heads": cfg.q_heads,
            "kv_heads": cfg.kv_heads, "head_dim": cfg.head_dim, "block_size": BS,
            "kv_dtype": cfg.kv_dtype, "q_dtype": cfg.q_dtype,
            "context_lens": list(cfg.lengths),
            "partition_size": first.partition_size,
            "shared_prompt_tokens": cfg.share_prefix_tokens,
            "shared_prefix": ({"groups": first.batch.plan.num_groups,
                               "members": int(first.batch.plan.group_offsets[-1]),
                               "blocks": first.batch.plan.group_blocks.tolist()}
                              if first.batch.plan is not None else None),
            "append": "fused into decode" if fused else "separate kernel",
            "replicas": reps, "pool_bytes_per_replica": pool_bytes,
            "kv_bytes_per_step": int(sum(kv_bytes) / reps),
            "kv_unique_bytes_per_step": int(sum(kv_unique) / reps),
            "seed": args.seed,
        },
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "seqs_per_s": round(cfg.batch / (ms_per_step * 1e-3), 1),
        "gpu_ms_per_step": round(gpu_ms_per_step, 5),
        "kernel_us": {"decode": round(decode_us, 3), "append_separate": round(append_us, 3),
                      "reduce": round(reduce_us, 3),
                      "decode_p10_p50_p90": [round(float(np.percentile(call_us, q)), 3)
                                             for q in (10, 50, 90)]},
        "algorithmic_flops_per_step": int(4 * sum(int(w.lens.astype(np.int64).sum())
                                                  for w in ws) / reps * cfg.q_heads
                                          * cfg.head_dim * cfg.layers),
        "roofline": {
            "bound": "hbm",
            "kernel": decode_kernel_name(cfg, first),
            "achieved": round(decode_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(decode_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(traffic_key(cfg, first, args)),
            "algorithmic_bytes": int(per_layer_unique),
        },
    }
    if args.window:
        result["window"] = [window_rate(ws, int(x), args.steps, stream, fused,
                                        decode_us + reduce_us)
                            for x in args.window.split(",")]
    if args.serve > 0:
        groups = tuple(int(x) for x in args.serve_prefix.split(",")) if args.serve_prefix else (0, 0)
        shared = {None: False, "on": True, "auto": "auto"}[args.serve_shared_prefix]
        result["serving"] = serving_rate(cfg, args.serve, stream, groups, args.serve_caching,
                                         args.serve_swap, args.serve_blocks, args.serve_gen,
                                         args.serve_window, shared)
    if args.swap > 0:
        result["swap"] = swap_rate(cfg, args.swap, args.steps, stream)
    if args.block_copy > 0:
        result["block_copy"] = block_copy_rate(cfg, args.block_copy, args.steps, stream)
    if args.gather_probe:
        result["gather_probe"] = gather_probe(stream)
    if args.workload == "llama13b_layer" and not args.no_other_configs:
        # The other workloads, each in its default form (their replicas are
        # built after the 13B ones are released to torch's cache).
        keep = first if not args.no_cpu_baseline else None
        for w in ws:
            if w is not keep:
                w.cache.close()
        ws = None
        result["other_configs"] = {name: config_summary(name, args.seed, wu, st, stream)
                                   for name, wu, st in OTHER_CONFIGS}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(first, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
