"""The five decode-step workloads.

Shapes come from the TontaubeV1 page (12.5 Hz frames; codebooks of 16,384
semantic and 4,096 acoustic entries, "codec" paragraph of the model section;
later stages greedy) and from the speculative-decoding blog (K draft tokens
verified in one target pass; 16-token KV blocks, "Dynamic Token-Level
Batching" section).  Value distributions list the standard deviation.
"""

from __future__ import annotations

import dataclasses
import math


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    index: int              # 1-based; the seed is 1000 + index (+ 100000 per trial)
    B: int                  # streams
    Kq: int                 # queries per stream (= rows appended per step)
    H_q: int
    H_kv: int
    D: int
    dtype: str              # "f32" or "bf16": q, K, V, o, h and W share it
    kv_len_dist: tuple      # ("fixed", n) | ("uniform", lo, hi) | ("loguniform", lo, hi)
    V: int                  # codebook (vocabulary) size
    G: int                  # number of codebook heads (grouped by stage)
    qkv_std: float
    w_std: float
    temperature: float      # 0 = greedy
    mode: str               # "greedy" | "sample" | "spec"
    block_size: int = 16
    draft_logit_std: float = 2.0
    description: str = ""
    trial: int = 0          # independent redraws of the same workload (0: the standard draw)

    @property
    def d_model(self) -> int:
        return self.H_q * self.D

    @property
    def M(self) -> int:
        return self.B * self.Kq

    @property
    def seed(self) -> int:
        return 1000 + self.index + 100000 * self.trial

    @property
    def workload(self) -> str:
        """Workload name built from what the step is and its sizes."""
        kind, *args = self.kv_len_dist
        lens = f"{kind}{'-'.join(str(a) for a in args)}"
        head = f"v{self.V}" + (f"x{self.G}heads" if self.G > 1 else "")
        return (f"decode_b{self.B}_q{self.Kq}_h{self.H_q}x{self.H_kv}_d{self.D}_{self.dtype}"
                f"_kv{lens}_{head}_{self.mode}")

    def expected_kv_tokens(self) -> float:
        kind, *args = self.kv_len_dist
        if kind == "fixed":
            return float(args[0])
        if kind == "uniform":
            return (args[0] + args[1]) / 2.0
        lo, hi = args
        # E[floor(exp(U))] ~ (hi - lo) / ln(hi / lo) - 1/2
        return (hi - lo) / math.log(hi / lo) - 0.5


_C1 = DecodeConfig(
    name="c1_tiny", index=1, B=1, Kq=1, H_q=4, H_kv=4, D=64, dtype="f32",
    kv_len_dist=("fixed", 64), V=4096, G=1, qkv_std=1.0 / 16.0, w_std=1.0 / 16.0,
    temperature=0.0, mode="greedy",
    description="tiny CPU-checkable step: d_model 256, 4/4 heads, D 64, 64 keys, fp32, greedy")
_C2 = DecodeConfig(
    name="c2_semantic", index=2, B=16, Kq=1, H_q=16, H_kv=8, D=128, dtype="bf16",
    kv_len_dist=("uniform", 100, 1500), V=16384, G=1, qkv_std=1.0, w_std=0.02,
    temperature=0.7, mode="sample",
    description="semantic stage: 16 streams, head 2048->16384, T=0.7 sampling")
_C3 = DecodeConfig(
    name="c3_mixed_acoustic", index=3, B=64, Kq=1, H_q=16, H_kv=8, D=128, dtype="bf16",
    kv_len_dist=("uniform", 200, 3000), V=4096, G=3, qkv_std=1.0, w_std=0.02,
    temperature=0.0, mode="greedy",
    description="mixed acoustic stages 1-3: 64 streams, 3 grouped 2048->4096 heads, greedy")
_C4 = DecodeConfig(
    name="c4_speculative", index=4, B=32, Kq=6, H_q=16, H_kv=8, D=128, dtype="bf16",
    kv_len_dist=("uniform", 300, 2000), V=4096, G=1, qkv_std=1.0, w_std=0.02,
    temperature=0.7, mode="spec",
    description="speculative verification: 32 streams x 6-query causal block, head 2048->4096")
_C5 = DecodeConfig(
    name="c5_high_concurrency", index=5, B=256, Kq=1, H_q=16, H_kv=8, D=128, dtype="bf16",
    kv_len_dist=("loguniform", 64, 8192), V=16384, G=1, qkv_std=1.0, w_std=0.02,
    temperature=0.0, mode="greedy",
    description="high concurrency: 256 streams, log-uniform KV 64..8192, head 2048->16384, greedy")

CONFIGS = {c.index: c for c in (_C1, _C2, _C3, _C4, _C5)}


def get_config(key) -> DecodeConfig:
    if isinstance(key, DecodeConfig):
        return key
    if isinstance(key, int):
        return CONFIGS[key]
    for c in CONFIGS.values():
        if key in (c.name, c.name.split("_")[0]):
            return c
    raise KeyError(key)
