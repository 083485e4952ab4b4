"""The five workload shapes and their scaled-down parity versions."""

from dataclasses import dataclass, replace
from typing import Optional


@dataclass(frozen=True)
class Config:
    name: str
    layers: int
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    kv_dtype: str            # "f16" | "bf16" | "e4m3"
    q_dtype: str             # "f16" | "bf16"
    lengths: tuple           # ("uniform", lo, hi) | ("const", L) | ("lognormal", median, sigma, lo, hi)
    pool_blocks: Optional[int] = None   # None: exactly the blocks the batch needs
    share_prefix_tokens: int = 0        # > 0: even-indexed sequences share this many tokens
    partition_size: int = 0             # default split-K partition (0: one pass)
    balanced: bool = True               # single pass: balanced over waves (else per sequence)
    shared_prefix: object = False       # False, True, "l2" or "auto" (see DecodeBatch)

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def src_dtype(self) -> str:
        """dtype of the K/V handed to the append step."""
        return self.q_dtype if self.kv_dtype == "e4m3" else self.kv_dtype


CONFIGS = {
    # 1 layer, batch 4, 4 query = 4 kv heads, dim 64, lengths U{1..200}, pool of
    # 64 blocks in shuffled order, one append per sequence.
    "tiny": Config("tiny", 1, 4, 4, 4, 64, "f16", "f16", ("uniform", 1, 200), pool_blocks=64,
                   balanced=False),
    # Llama-2-13B-shaped layer: MHA 40 x 128, batch 32, lengths U{128..2048}, pool
    # sized to the batch with randomly permuted blocks.
    "llama13b_layer": Config("llama13b_layer", 1, 32, 40, 40, 128, "f16", "f16",
                             ("uniform", 128, 2048), balanced=False),
    # 7B-class full decode step: 32 layers, MHA 32 x 128, batch 64, every context
    # 2048 tokens (about 1.07 GB of KV per request, about 68.7 GB of pool).
    "7b_32layer": Config("7b_32layer", 32, 64, 32, 32, 128, "f16", "f16", ("const", 2048)),
    # GQA 64 query / 8 kv heads x 128 in bf16, batch 128, lengths log-normal
    # (median 1000) clipped to [16, 8192]; half the sequences share a 512-token
    # prefix through refcounted blocks.
    # The batch reads the shared blocks in the form "auto" picks for it (here
    # through the L2 by the balanced pass; the prefix kernel for long prompts).
    "gqa_prefix": Config("gqa_prefix", 1, 128, 64, 8, 128, "bf16", "bf16",
                         ("lognormal", 1000.0, 1.0, 16, 8192), share_prefix_tokens=512,
                         shared_prefix="auto"),
    # Long-context split-K: batch 8, MHA 32 x 128, lengths U{16384..32768}, KV in
    # FP8 E4M3 with per-head fp32 scales, q fp16, partitions of 512 tokens.
    "longctx_fp8": Config("longctx_fp8", 1, 8, 32, 32, 128, "e4m3", "f16",
                          ("uniform", 16384, 32768), partition_size=512),
}


def scaled(name: str) -> Config:
    """A parity-test version of a workload: same structure, sizes the oracle
    finishes in seconds, still several tiles and partitions with ragged tails."""
    c = CONFIGS[name]
    if name == "tiny":
        return c
    if name == "llama13b_layer":
        return replace(c, name="llama13b_layer_small", batch=6, q_heads=5, kv_heads=5,
                       lengths=("uniform", 128, 700))
    if name == "7b_32layer":
        return replace(c, name="7b_32layer_small", layers=3, batch=4, q_heads=4, kv_heads=4,
                       lengths=("const", 2048))
    if name == "gqa_prefix":
        return replace(c, name="gqa_prefix_small", batch=8, q_heads=16, kv_heads=2,
                       lengths=("lognormal", 300.0, 1.0, 16, 1200), share_prefix_tokens=512)
    if name == "longctx_fp8":
        return replace(c, name="longctx_fp8_small", batch=3, q_heads=3, kv_heads=3,
                       lengths=("uniform", 1100, 2600))
    raise KeyError(name)
