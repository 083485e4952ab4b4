"""Seeded request traces for the continuous-batching loop.

[P2] "连续批处理：别再等最慢的那个请求了": requests arrive while others run,
finish after different numbers of generated tokens, and a finished request
leaves the batch at once. A request may ask for several samples of one
prompt (beam search, parallel sampling: "PagedAttention：..." lets them share
the prompt's blocks). Only the inputs are drawn here: arrival iteration,
prompt length, generated length, number of samples; and the K, V and q rows
the loop feeds the cache, keyed by what they stand for.
"""

from dataclasses import dataclass

import numpy as np

from .gen import normal, seed_for


@dataclass(frozen=True)
class RequestSpec:
    rid: int
    arrival: int      # iteration at which it joins the waiting queue
    prompt_len: int   # tokens written to the cache on admission
    gen_len: int      # decode steps per sample
    samples: int      # sequences sharing the prompt
    block_keys: tuple = ()  # content keys of the prompt's full blocks (prefix caching)


def _key(*parts) -> int:
    """A 64-bit name for a block's contents (what a hash of its tokens and
    every token before them would be)."""
    return seed_for("block", 0, *parts) | 1


def request_trace(name: str, seed: int, num_requests: int, max_prompt: int, max_gen: int,
                  mean_gap: float = 1.0, multi_sample: float = 0.3, max_samples: int = 3,
                  prefix_groups: int = 0, shared_tokens: int = 0):
    """prefix_groups > 0: each request belongs to one of that many groups (or,
    with probability 1 / (groups + 1), to none); the first shared_tokens
    tokens of a grouped request's prompt are its group's (a system prompt),
    so the keys of those full blocks are the group's."""
    rng = np.random.Generator(np.random.PCG64(seed_for(name, seed, "requests")))
    t = 0.0
    out = []
    for rid in range(num_requests):
        t += rng.exponential(mean_gap)
        samples = int(rng.integers(2, max_samples + 1)) if rng.random() < multi_sample else 1
        plen = int(rng.integers(1, max_prompt + 1))
        gen = int(rng.integers(1, max_gen + 1))
        group = int(rng.integers(-1, prefix_groups)) if prefix_groups > 0 else -1
        if group >= 0:
            plen = max(plen, shared_tokens)
        keys = []
        for j in range(plen // 16):
            if group >= 0 and (j + 1) * 16 <= shared_tokens:
                keys.append(_key(name, seed, "group", group, j))
            else:
                keys.append(_key(name, seed, "request", rid, j))
        out.append(RequestSpec(rid, int(t), plen, gen, samples, tuple(keys)))
    return out


def prompt_rows(name: str, seed: int, rid: int, layer: int, which: str, n: int, kv_heads: int,
                head_dim: int, dtype: str, device):
    """K or V rows [n, Hkv, D] of request rid's prompt."""
    return normal((n, kv_heads, head_dim), dtype, seed_for(name, seed, "prompt", rid, layer, which),
                  device)


def keyed_prompt_rows(name: str, seed: int, spec: RequestSpec, layer: int, which: str,
                      kv_heads: int, head_dim: int, dtype: str, device):
    """K or V rows [prompt_len, Hkv, D] of a request whose full blocks carry
    content keys: the rows of each full block are drawn from its key (equal
    keys, equal contents), those of the partial last block from the request."""
    import torch
    parts = [normal((16, kv_heads, head_dim), dtype, seed_for(name, seed, "block", k, layer, which),
                    device) for k in spec.block_keys]
    tail = spec.prompt_len - 16 * len(spec.block_keys)
    if tail or not parts:
        parts.append(normal((tail, kv_heads, head_dim), dtype,
                            seed_for(name, seed, "tail", spec.rid, layer, which), device))
    return torch.cat(parts, dim=0)


def step_rows(name: str, seed: int, it: int, layer: int, which: str, n: int, heads: int,
              head_dim: int, dtype: str, device):
    """Rows [n, heads, D] for the n running sequences of iteration it: the new
    token's K or V (which = "k", "v"), or the query (which = "q")."""
    return normal((n, heads, head_dim), dtype, seed_for(name, seed, "step", it, layer, which),
                  device)
