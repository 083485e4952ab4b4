"""Seeded synthetic inputs for the paged KV cache hot path.

This module only draws inputs: context lengths, the random order in which
blocks are returned to the pool (random physical placement), which sequences
share a prompt prefix, and N(0,1) query / key / value tensors rounded to
their storage dtype. It holds none of the method's arithmetic (no paging, no
attention, no quantisation) and imports neither the library nor the oracle;
both sides consume what it produces.

The workloads stand in for the serving cases of the pages (a Llama-2-13B
class model served on one GPU, and a 32-layer, 32-head, head_dim-128 7B-class
model at 2048 tokens: "vLLM 推理加速原理详解：大模型服务吞吐量为何能提升 10 倍",
sections "真正吃显存的是 KV Cache，不是模型权重" and "连续批处理：别再等最慢的那个请求了");
the pages' serving benchmark uses prompts and model weights that are not
used here.
"""

from .configs import CONFIGS, Config, scaled  # noqa: F401
from .requests import (RequestSpec, keyed_prompt_rows, prompt_rows, request_trace,  # noqa: F401
                       step_rows)
from .gen import (  # noqa: F401
    context_lengths,
    fp8_scales,
    free_order,
    kv_tokens,
    normal,
    q_tensor,
    seed_for,
    sharers,
)
