"""GPU parity of kv_cache_append on its own, through the C ABI.

* Slots < 0 and slots past the pool (num_blocks * 16 and beyond) are skipped:
  among valid slots in random order they leave the whole pool, compared byte
  for byte with the oracle's append of the valid slots only, untouched.
* The FP8 store, exhaustively: every finite fp16 (and every finite bf16) bit
  pattern is appended as K and as V under several per-head scales (tiny
  ones that saturate most inputs, 1, and large ones that push most inputs
  into the subnormals or to zero), and the stored bytes must equal the
  oracle's encoder (pinned to the format definition and to torch's
  float8_e4m3fn) for every one.
"""

import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_450_amd as P
import workloads as W
from oracle import pool as opool
from paged_kv_cache_450_amd.runtime import PagedKVCache
from tests import harness as H

pytestmark = pytest.mark.gpu
BS = 16


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(autouse=True)
def _gpu(require_gpu):
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("kv,hkv,dim", [("f16", 2, 64), ("bf16", 4, 128), ("e4m3", 2, 128)])
def test_append_skips_negative_and_out_of_range_slots(kv, hkv, dim):
    say(f"append slot skipping {kv} Hkv={hkv} D={dim}")
    src = "f16" if kv == "e4m3" else kv
    layers, nb = 2, 12
    rng = np.random.default_rng(W.seed_for("append_skip", 0, kv, hkv, dim))
    cache = PagedKVCache(layers, nb, hkv, dim, kv, "cuda", fill_byte=H.POISON)
    n_slots = nb * BS
    valid = rng.permutation(n_slots)[:70]
    bad = np.array([-1, -5, -(1 << 40), n_slots, n_slots + 1, n_slots + 1000, 1 << 40])
    slots = np.concatenate([valid, bad])
    rng.shuffle(slots)
    T = slots.size
    k = W.normal((T, hkv, dim), src, W.seed_for("append_skip", 1, kv), "cuda")
    v = W.normal((T, hkv, dim), src, W.seed_for("append_skip", 2, kv), "cuda")
    ks = vs = ks_np = vs_np = None
    if kv == "e4m3":
        ks, vs = W.fp8_scales([k]), W.fp8_scales([v])
        ks_np, vs_np = ks.cpu().numpy(), vs.cpu().numpy()
    host = np.full(opool.pool_bytes(layers, nb, BS, hkv, dim, kv), H.POISON, dtype=np.uint8)
    p6 = opool.view_pool(host, layers, nb, BS, hkv, dim, kv)
    keep = (slots >= 0) & (slots < n_slots)
    for layer in range(layers):
        P.kv_cache_append(cache.handle, layer, k, v, torch.from_numpy(slots.astype(np.int64)).cuda(),
                          ks, vs)
        opool.append(p6, layer, H.raw16(k)[keep], H.raw16(v)[keep], src, kv, slots[keep], ks_np,
                     vs_np)
    torch.cuda.synchronize()
    got = cache.buf.cpu().numpy()
    if not np.array_equal(got, host):
        bad_at = np.flatnonzero(got != host)
        raise AssertionError(f"{bad_at.size} pool bytes differ, first {bad_at[:4]}")
    cache.close()


def finite_rows(src, dim):
    """Every finite bit pattern of the 16-bit source type, as rows [T, 1, dim]
    (the last row padded with zeros)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if src == "f16":
        finite = (bits & 0x7C00) != 0x7C00
    else:
        finite = (bits & 0x7F80) != 0x7F80
    vals = bits[finite]
    T = -(-vals.size // dim)
    out = np.zeros(T * dim, dtype=np.uint16)
    out[:vals.size] = vals
    return out.reshape(T, 1, dim), vals.size


@pytest.mark.parametrize("src", ["f16", "bf16"])
def test_fp8_append_is_exhaustively_exact(src):
    dim = 128
    rows, n = finite_rows(src, dim)
    T = rows.shape[0]
    nb = -(-T // BS)
    say(f"fp8 append exhaustive from {src}: {n} finite values")
    tdt = H.TORCH_DTYPES[src]
    k = torch.from_numpy(rows.view(np.int16)).view(tdt).cuda()
    v = torch.from_numpy(rows[::-1].copy().view(np.int16)).view(tdt).cuda()
    slots = np.arange(T, dtype=np.int64)
    for sc in (1.0 / 65536, 1.0 / 448, 0.37, 1.0, 3.0, 448.0, 65504.0):
        cache = PagedKVCache(1, nb, 1, dim, "e4m3", "cuda", fill_byte=H.POISON)
        ks = torch.tensor([sc], dtype=torch.float32, device="cuda")
        vs = torch.tensor([sc * 0.75], dtype=torch.float32, device="cuda")
        P.kv_cache_append(cache.handle, 0, k, v, torch.from_numpy(slots).cuda(), ks, vs)
        torch.cuda.synchronize()
        host = np.full(opool.pool_bytes(1, nb, BS, 1, dim, "e4m3"), H.POISON, dtype=np.uint8)
        p6 = opool.view_pool(host, 1, nb, BS, 1, dim, "e4m3")
        opool.append(p6, 0, rows, rows[::-1], src, "e4m3", slots, ks.cpu().numpy(),
                     vs.cpu().numpy())
        got = cache.buf.cpu().numpy()
        if not np.array_equal(got, host):
            bad = np.flatnonzero(got != host)
            raise AssertionError(f"scale {sc}: {bad.size} stored bytes differ, first {bad[:4]}")
        cache.close()
