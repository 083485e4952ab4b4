"""Seeded random shapes through every decode form, against the oracle.

Each case draws a batch (1-48 sequences, 1-2 layers), a head layout (kv heads
1-8, group 1, 2, 4 or 8, head_dim 64 or 128), a cache dtype (fp16, bf16 or
FP8 E4M3 with an fp16 or bf16 query), a length range, and a decode form the
library offers for it: the per-sequence or the balanced single pass, split-K
at 16-256 tokens, the shared-prefix kernel pass or the L2 form over even
sequences that share a prompt, each as the fused step or as separate append
and decode calls. The whole pool is compared byte for byte after the appends
and every output of every layer against the oracle. The cases are fixed by
their seeds, so a failure names a reproducible case."""

import sys

import numpy as np
import pytest
import torch

import workloads as W
from tests import harness as H

def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture
def _gpu(require_gpu):
    yield
    torch.cuda.synchronize()


def draw_case(seed: int):
    """One configuration and its decode form, from the seed alone."""
    r = np.random.default_rng(np.random.PCG64(1_000_003 + seed))
    kv = ["f16", "bf16", "e4m3"][r.integers(3)]
    q = kv if kv != "e4m3" else ["f16", "bf16"][r.integers(2)]
    hkv = int(r.choice([1, 2, 4, 8]))
    g = int(r.choice([1, 2, 4, 8]))
    dim = int(r.choice([64, 128]))
    batch = int(r.integers(1, 49))
    layers = int(r.integers(1, 3))
    hi = int(r.choice([16, 40, 300, 1200]))
    lo = int(r.integers(1, hi + 1)) if r.random() < 0.3 else 1
    ps = 0 if r.random() < 0.5 else int(r.choice([16, 64, 256]))
    balanced = kv != "e4m3" and ps == 0 and r.random() < 0.6
    share = 0
    shared = None
    if balanced and batch >= 4 and r.random() < 0.5:
        share = int(r.choice([16, 32, 64]))
        shared = [True, "l2"][r.integers(2)]
    fused = bool(r.random() < 0.7)
    cfg = W.Config(f"rand{seed}", layers, batch, hkv * g, hkv, dim, kv, q, ("uniform", lo, hi),
                   share_prefix_tokens=share, partition_size=ps, balanced=balanced)
    return cfg, fused, shared


CASES = list(range(64))


@pytest.mark.gpu
@pytest.mark.parametrize("seed", CASES)
def test_random_shape_matches_oracle(seed, _gpu):
    from tests.test_gpu_parity import check_bookkeeping, check_layers

    cfg, fused, shared = draw_case(seed)
    say(f"random shape {seed}: B={cfg.batch} layers={cfg.layers} Hq={cfg.q_heads} "
        f"Hkv={cfg.kv_heads} D={cfg.head_dim} kv={cfg.kv_dtype} q={cfg.q_dtype} "
        f"lens={cfg.lengths} ps={cfg.partition_size} balanced={cfg.balanced} "
        f"share={cfg.share_prefix_tokens} shared={shared} fused={fused}")
    side = H.build_product(cfg, seed=seed, fused=fused, shared_prefix=shared)
    torch.cuda.synchronize()
    o = H.oracle_bookkeeping(cfg, seed)
    check_bookkeeping(side, o)
    check_layers(cfg, side, o, list(range(cfg.batch)), range(cfg.layers), whole_pool=True)


def test_cases_cover_every_form():
    """The fixed seeds reach each form at least once (host only)."""
    forms = set()
    for seed in CASES:
        cfg, fused, shared = draw_case(seed)
        forms.add(("fp8" if cfg.kv_dtype == "e4m3" else "16bit",
                   "splitk" if cfg.partition_size else
                   ("balanced" if cfg.balanced else "perseq")))
        if shared is not None:
            forms.add(("shared", str(shared)))
        forms.add(("fused", fused))
    need = {("16bit", "perseq"), ("16bit", "balanced"), ("16bit", "splitk"),
            ("fp8", "perseq"), ("fp8", "splitk"), ("shared", "True"), ("shared", "l2"),
            ("fused", True), ("fused", False)}
    assert need <= forms, need - forms


# kv head counts that are not powers of two: the balanced pass takes them in
# head groups of 4 (or 8 on the vector path), 2 or 1, with group sizes the
# fixed seeds above never reach (3 heads: groups of 1; 6: of 2; 12: of 4; 40:
# of 8 on the vector path). Batches small enough that waves outnumber tiles
# (one tile per range) and large enough that ranges hold many.
HEAD_COUNTS = [(3, 1, 4), (5, 1, 24), (6, 1, 24), (6, 8, 24), (12, 1, 24), (12, 2, 24),
               (12, 8, 6), (10, 4, 24), (40, 1, 24)]


@pytest.mark.gpu
@pytest.mark.parametrize("hkv,g,batch", HEAD_COUNTS)
def test_balanced_pass_with_any_head_count(hkv, g, batch, _gpu):
    from tests.test_gpu_parity import check_bookkeeping, check_layers

    seed = 500 + hkv * 10 + g
    cfg = W.Config(f"heads{hkv}x{g}", 1, batch, hkv * g, hkv, 128, "bf16", "bf16",
                   ("uniform", 1, 700), balanced=True)
    say(f"balanced head count: Hkv={hkv} G={g} B={batch} seed={seed}")
    side = H.build_product(cfg, seed=seed, fused=True)
    torch.cuda.synchronize()
    o = H.oracle_bookkeeping(cfg, seed)
    check_bookkeeping(side, o)
    check_layers(cfg, side, o, list(range(cfg.batch)), range(cfg.layers), whole_pool=True)


# The vector-ALU balanced pass (one query head per kv head: the LDS tile ring)
# in each of its instances: fused step or not, head_dim 64 or 128, plain,
# shared blocks through the L2, or after the prefix kernel.
VALU_FORMS = [(fused, dim, shared, kv) for fused in (True, False) for dim in (64, 128)
              for shared, kv in ((None, "f16"), ("l2", "bf16"), (True, "f16"))]


@pytest.mark.gpu
@pytest.mark.parametrize("fused,dim,shared,kv", VALU_FORMS)
def test_vector_balanced_pass_forms(fused, dim, shared, kv, _gpu):
    from tests.test_gpu_parity import check_bookkeeping, check_layers

    seed = 900 + dim + (7 if fused else 0) + (3 if shared == "l2" else 5 if shared else 0)
    cfg = W.Config(f"valu{dim}", 2, 20, 6, 6, dim, kv, kv, ("uniform", 1, 900),
                   share_prefix_tokens=48 if shared is not None else 0, balanced=True)
    say(f"vector balanced: fused={fused} D={dim} shared={shared} kv={kv} seed={seed}")
    side = H.build_product(cfg, seed=seed, fused=fused, shared_prefix=shared)
    torch.cuda.synchronize()
    o = H.oracle_bookkeeping(cfg, seed)
    check_bookkeeping(side, o)
    check_layers(cfg, side, o, list(range(cfg.batch)), range(cfg.layers), whole_pool=True)
