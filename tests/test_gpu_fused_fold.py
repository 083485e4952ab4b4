"""The balanced pass of the fused step (paged_attn_decode_append with a
workspace): the streaming kernel reads each context's blocks without the new
token's position and the token as one more tile from its source rows, and
the wave that reads that tile stores it to its slot. Checked against the
oracle, and the pool against the oracle's appends byte for byte, beside the
same step as kv_cache_append + paged_attn_decode, on batches that mix
contexts read whole by one wave with contexts split between waves (and new
tokens whose tile falls in another wave than their block), a context that is
only its new token, new tokens that open a block, and a sequence whose last
block id lies outside the pool (no store, and that block's tokens are absent
from its attention)."""

import sys

import numpy as np
import pytest
import torch

import workloads as W
from tests import harness as H

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(autouse=True)
def _gpu(require_gpu):
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("dt,hq,hkv,dim,hi", [
    ("f16", 8, 8, 128, 40),     # one query head per kv head, short contexts
    ("bf16", 32, 8, 128, 600),  # four per kv head (matrix cores), whole and split contexts
    ("f16", 16, 2, 64, 600),    # eight per kv head, D = 64
    ("bf16", 4, 2, 64, 300),    # two per kv head
    ("f16", 16, 2, 64, 40),     # eight per kv head, short contexts
])
def test_fused_step_folds_new_tokens_in_merge(dt, hq, hkv, dim, hi):
    import paged_kv_cache_450_amd as P
    from oracle import attention as oattn

    B = 48
    cfg = W.Config(f"fold_{dt}_{hq}_{hkv}_{dim}_{hi}", 1, B, hq, hkv, dim, dt, dt,
                   ("uniform", 1, hi))

    def covers(lens):  # the cases named above
        return (((lens == 1).any() or hi > 40) and ((lens % 16 == 1) & (lens > 1)).any()
                and ((lens > 16) & (lens % 16 > 1)).any())
    seed = next(s for s in range(100) if covers(W.context_lengths(cfg, s)))
    say(f"fused fold {cfg.name} seed={seed}")
    side = H.build_product(cfg, seed=seed, balanced=True, run_step=False)
    b = side.batch
    o = H.oracle_bookkeeping(cfg, seed)
    lens = side.lens.copy()
    assert covers(lens)
    bad = next(i for i in range(B) if lens[i] > 16 and lens[i] % 16 > 1)
    tables = b.tables.clone()
    tables[bad, (int(lens[bad]) - 1) // 16] = -1
    lens_dev = torch.from_numpy(lens).cuda()
    max_ctx = int(lens.max())
    wsb = P.paged_attn_workspace_bytes(B, hq, dim, max_ctx, 0)
    ws = torch.empty(wsb // 4, dtype=torch.float32, device="cuda")
    slots = o.slots_new.astype(np.int64).copy()
    slots[bad] = -1  # kv_cache_append skips it, as the fused step must
    slots_dev = torch.from_numpy(slots).cuda()
    outs = {}
    before = side.cache.buf.clone()
    for form in ("fused", "separate"):
        say(f"  form={form}")
        side.cache.buf.copy_(before)
        out = torch.full_like(b.out, float("nan"))
        if form == "fused":
            P.paged_attn_decode_append(side.cache.handle, 0, side.k_new[0], side.v_new[0],
                                       side.q[0], out, tables, lens_dev, b.scale, max_ctx, 0, ws)
        else:
            P.kv_cache_append(side.cache.handle, 0, side.k_new[0], side.v_new[0], slots_dev)
            P.paged_attn_decode(side.cache.handle, 0, side.q[0], out, tables, lens_dev, b.scale,
                                max_ctx, 0, ws)
        torch.cuda.synchronize()
        outs[form] = H.out_f64(out, dt)
        # the pool: every sequence's new token stored but the one with the bad id
        p6 = H.expected_layer_pool(cfg, side, o, 0, range(B))
        blk, off = int(o.slots_new[bad]) // 16, int(o.slots_new[bad]) % 16
        p6[0][:, blk, :, off, :] = np.full(p6.itemsize, H.POISON, np.uint8).view(p6.dtype)[0]
        nb = side.cache.num_blocks
        got = H.gpu_layer_blocks(cfg, side, 0, np.arange(nb))
        assert np.array_equal(got.view(np.uint8), p6[0].view(np.uint8)), form

    q = H.q_f64(side.q[0], dt)
    ref_lens = lens.copy()
    ref_lens[bad] = (int(lens[bad]) - 1) // 16 * 16  # its last block is absent
    ref = oattn.paged_decode(p6, 0, q, o.tables, ref_lens, float(np.float32(b.scale)), dt)
    for form, got in outs.items():
        H.assert_close(got, ref, dt, f"fused fold, {form}")
