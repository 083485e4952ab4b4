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


def request_trace(name: str, seed: int, num_requests: int, max_prompt: int, max_gen: int,
                  mean_gap: float = 1.0, multi_sample: float = 0.3, max_samples: int = 3):
    rng = np.random.Generator(np.random.PCG64(seed_for(name, seed, "requests")))
    t = 0.0
    out = []
    for rid in range(num_requests):
        t += rng.exponential(mean_gap)
        samples = int(rng.integers(2, max_samples + 1)) if rng.random() < multi_sample else 1
        out.append(RequestSpec(rid, int(t), int(rng.integers(1, max_prompt + 1)),
                               int(rng.integers(1, max_gen + 1)), samples))
    return out


def prompt_rows(name: str, seed: int, rid: int, layer: int, which: str, n: int, kv_heads: int,
                head_dim: int, dtype: str, device):
    """K or V rows [n, Hkv, D] of request rid's prompt."""
    return normal((n, kv_heads, head_dim), dtype, seed_for(name, seed, "prompt", rid, layer, which),
                  device)


def step_rows(name: str, seed: int, it: int, layer: int, which: str, n: int, heads: int,
              head_dim: int, dtype: str, device):
    """Rows [n, heads, D] for the n running sequences of iteration it: the new
    token's K or V (which = "k", "v"), or the query (which = "q")."""
    return normal((n, heads, head_dim), dtype, seed_for(name, seed, "step", it, layer, which),
                  device)
