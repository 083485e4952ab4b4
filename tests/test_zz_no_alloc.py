"""paged_attn_decode_append_noalloc, the decode step for callers that cannot
allocate: its workspace is the library's static device scratch. Through the C
ABI, its output must equal paged_attn_decode_append's with a caller
workspace (the same kernels run), bit for bit, and match the oracle; two
calls in a row, the second on a smaller batch, so the second call finds the
first one's partials in the scratch. A batch whose workspace would exceed the
scratch is refused before anything runs.
"""

import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_450_amd as P
import workloads as W
from tests import harness as H
from tests.test_gpu_parity import check_bookkeeping

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(autouse=True)
def _gpu(require_gpu):
    yield
    torch.cuda.synchronize()


def run_both(cfg, seed):
    """One fused decode step of layer 0 through both entry points on the same
    cache: the existing call with a caller workspace (then the reduce when
    split-K), and the no-alloc call. Returns (side, existing out, no-alloc out)."""
    side = H.build_product(cfg, seed=seed, run_step=False)
    b = side.batch
    ks, vs = side.k_scale[0], side.v_scale[0]
    ps = b.partition_size
    ref_out = torch.full_like(b.out, float("nan"))
    ws = b.workspace
    if ws is None:  # per-sequence forms get a workspace only for the comparison's sake
        ws = torch.empty(max(P.paged_attn_workspace_bytes(cfg.batch, cfg.q_heads, cfg.head_dim,
                                                          b.max_context_len, 0), 16) // 4,
                         dtype=torch.float32, device="cuda")
    P.paged_attn_decode_append(side.cache.handle, 0, side.k_new[0], side.v_new[0], side.q[0],
                               None if ps else ref_out, b.tables, b.lens, b.scale,
                               b.max_context_len, ps, ws, ks, vs)
    if ps:
        P.paged_attn_reduce(ws, ref_out, b.lens, b.max_context_len, ps)
    got = torch.full_like(b.out, float("nan"))
    P.paged_attn_decode_append_noalloc(side.cache.handle, 0, side.k_new[0], side.v_new[0],
                                       side.q[0], got, b.tables, b.lens, b.scale,
                                       b.max_context_len, ps, ks, vs)
    torch.cuda.synchronize()
    return side, ref_out, got


CASES = [  # (workload, partition size, larger batch, smaller batch)
    ("longctx_fp8", 512, 3, 2),     # split-K on an FP8 cache, reduce inside the call
    ("llama13b_layer", 256, 6, 3),  # split-K, 16-bit, fused append in the kernel
    ("gqa_prefix", 0, 8, 5),        # balanced single pass (matrix cores), merge partials
    ("llama13b_layer", 0, 6, 2),    # balanced single pass (vector ALU)
    ("longctx_fp8", 0, 3, 1),       # FP8 single pass: per sequence, no scratch
]


@pytest.mark.parametrize("name,ps,big,small", CASES)
def test_noalloc_matches_the_workspace_call(name, ps, big, small):
    from dataclasses import replace

    base = W.scaled(name)
    for k, batch in enumerate((big, small)):
        cfg = replace(base, name=f"{base.name}_noalloc_{batch}", batch=batch, partition_size=ps)
        say(f"noalloc {cfg.name} B={batch} ps={ps} call {k + 1} of 2")
        side, ref_out, got = run_both(cfg, seed=13 + k)
        assert torch.equal(got.view(torch.int16), ref_out.view(torch.int16)), \
            f"{cfg.name}: no-alloc output differs from the workspace call"
        o = H.oracle_bookkeeping(cfg, 13 + k)
        check_bookkeeping(side, o)
        seqs = list(range(cfg.batch))
        p6 = H.expected_layer_pool(cfg, side, o, 0, seqs)
        ids = np.arange(o.model.num_blocks)
        assert np.array_equal(H.gpu_layer_blocks(cfg, side, 0, ids), p6[0][:, ids]), "pool bytes"
        ref = H.oracle_outputs(cfg, side, o, 0, p6, seqs)
        H.assert_close(H.out_f64(got, cfg.q_dtype), ref, cfg.kv_dtype, cfg.name)
        del side


def test_noalloc_refuses_a_batch_beyond_the_scratch():
    """Split-K partials of 64 sequences x 32 heads x 64 partitions need about
    68 MB, more than the 32 MiB scratch: refused with INVALID, nothing run."""
    cfg = W.Config("noalloc_too_big", 1, 64, 32, 32, 128, "f16", "f16", ("const", 32),
                   partition_size=16)
    side = H.build_product(cfg, seed=0, run_step=False)
    b = side.batch
    need = P.paged_attn_workspace_bytes(64, 32, 128, 64 * 16, 16)
    assert need > P.STATIC_SCRATCH_BYTES
    out = torch.full_like(b.out, float("nan"))
    with pytest.raises(P.PkvError) as e:
        P.paged_attn_decode_append_noalloc(side.cache.handle, 0, side.k_new[0], side.v_new[0],
                                           side.q[0], out, b.tables, b.lens, b.scale, 64 * 16,
                                           16)
    assert e.value.status == P.PKV_ERR_INVALID and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
