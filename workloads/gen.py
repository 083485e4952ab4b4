"""Seeded generators. Every draw is keyed by (workload name, seed, tags)."""

import hashlib
import math

import numpy as np
import torch

from .configs import Config

_TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}
_CHUNK = 1 << 27  # elements drawn per torch.randn call (bounds the fp32 temporary)


def seed_for(name: str, seed: int, *tags) -> int:
    """A 63-bit seed derived from the workload name, the user seed and tags."""
    h = hashlib.sha256(repr((name, int(seed)) + tuple(tags)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def context_lengths(cfg: Config, seed: int) -> np.ndarray:
    """Context length of every sequence, the new token included."""
    rng = np.random.Generator(np.random.PCG64(seed_for(cfg.name, seed, "lengths")))
    kind = cfg.lengths[0]
    if kind == "uniform":
        _, lo, hi = cfg.lengths
        lens = rng.integers(lo, hi + 1, size=cfg.batch)
    elif kind == "const":
        lens = np.full(cfg.batch, cfg.lengths[1])
    elif kind == "lognormal":
        _, median, sigma, lo, hi = cfg.lengths
        x = rng.lognormal(mean=math.log(median), sigma=sigma, size=cfg.batch)
        lens = np.clip(np.rint(x), lo, hi)
    else:
        raise ValueError(kind)
    lens = lens.astype(np.int64)
    if cfg.share_prefix_tokens:
        # Sharers keep at least one private token after the shared prefix, so
        # the new token never lands in a shared block.
        for i in sharers(cfg):
            lens[i] = max(lens[i], cfg.share_prefix_tokens + 1)
    return lens.astype(np.int32)


def sharers(cfg: Config) -> list:
    """Indices of the sequences that share the prompt prefix (the even ones)."""
    if not cfg.share_prefix_tokens:
        return []
    return list(range(0, cfg.batch, 2))


def free_order(num_blocks: int, name: str, seed: int) -> np.ndarray:
    """A random permutation of the block ids: the order in which they are
    handed back to a fresh pool, which fixes the random physical placement."""
    rng = np.random.Generator(np.random.PCG64(seed_for(name, seed, "placement")))
    return rng.permutation(num_blocks).astype(np.int32)


def _generator(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, dtype: str, seed: int, device) -> torch.Tensor:
    """N(0, 1) draws in fp32, rounded to nearest even into dtype."""
    device = torch.device(device)
    out = torch.empty(shape, dtype=_TORCH_DTYPES[dtype], device=device)
    flat = out.view(-1)
    g = _generator(device, seed)
    for start in range(0, flat.numel(), _CHUNK):
        n = min(_CHUNK, flat.numel() - start)
        flat[start:start + n] = torch.randn(n, generator=g, dtype=torch.float32, device=device)
    return out


def kv_tokens(cfg: Config, seed: int, layer: int, which: str, part: str, n_tokens: int,
              device) -> torch.Tensor:
    """K or V rows [n_tokens, Hkv, D] in the source dtype.

    part = "cached" for the tokens already in the cache before the decode step,
    "new" for the token the step appends (one per sequence).
    """
    assert which in ("k", "v") and part in ("cached", "new")
    return normal((n_tokens, cfg.kv_heads, cfg.head_dim), cfg.src_dtype,
                  seed_for(cfg.name, seed, "kv", layer, which, part), device)


def q_tensor(cfg: Config, seed: int, layer: int, device) -> torch.Tensor:
    return normal((cfg.batch, cfg.q_heads, cfg.head_dim), cfg.q_dtype,
                  seed_for(cfg.name, seed, "q", layer), device)


def fp8_scales(parts) -> torch.Tensor:
    """Per-kv-head fp32 scale = max |x| / 448 over the given [T, Hkv, D] tensors
    (the source rows of every token of the head, cached and new)."""
    amax = None
    for t in parts:
        if t.numel() == 0:
            continue
        a = t.abs().amax(dim=(0, 2)).to(torch.float32)
        amax = a if amax is None else torch.maximum(amax, a)
    return amax / 448.0
