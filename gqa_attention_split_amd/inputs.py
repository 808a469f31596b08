"""Seeded synthetic inputs for the GQA exp-sum-div graph.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic. Both the HIP path (tests, bench) and the CPU oracle take
their inputs from here, so the two sides see the same fp16 bits.

Shapes follow the GQA tutorial graph on the Mirage documentation page
("Mirage: Define GQA Computation Graph"): Q is (B, M, D), K is stored
head-dim-major as (B, D, N), V is (B, N, D), all fp16. The batch-scaled form
(axis 0 = 2 * batch_size, i.e. batch x 2 KV heads) is the one the kaispace
blog walks through in its section 1 ("entering from the GQA benchmark").

Recipe (same for every config): a numpy PCG64 generator seeded with the
config's seed draws, in this order, Q, then K (directly in its (B, D, N)
layout), then V, as float64 samples of the stated distribution; each array is
rounded to fp16 with round-to-nearest-even (numpy's float64 -> float16 cast).
The pages measure on no dataset; these draws stand in for the benchmark's
random tensors, with scores scaled so that exp stays in fp16 range (the graph
has no max subtraction).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

HEAD_DIM = 64


@dataclass(frozen=True)
class GqaConfig:
    name: str
    B: int          # batch x KV heads
    M: int          # query rows per KV head
    N: int          # keys
    qk_std: float   # Q and K ~ N(0, qk_std^2)
    v_dist: str     # "normal" (std 1) or "uniform" (U(-1, 1))
    seed: int
    D: int = HEAD_DIM

    @property
    def flops(self) -> int:
        """Two contractions, 2*B*M*N*D flops each (exp, sum, divide not counted)."""
        return 4 * self.B * self.M * self.N * self.D

    @property
    def algorithmic_bytes(self) -> int:
        """Q, K, V read once and O written once, all fp16."""
        return 2 * self.D * (2 * self.B * self.M + 2 * self.B * self.N)


# The workloads: the tutorial shape at batch 1 and batch 8, a long-KV case, a
# decode-like case with few query rows, a large-batch case, and the
# tutorial's launch example at head dim 128 (Q (64, 1, 128), K (64, 128, 4096),
# V (64, 4096, 128): one query row per KV head, i.e. decoding).
CONFIGS = {
    "gqa_b2_m256_n4096": GqaConfig("gqa_b2_m256_n4096", 2, 256, 4096, 0.25, "normal", 101),
    "gqa_b16_m256_n4096": GqaConfig("gqa_b16_m256_n4096", 16, 256, 4096, 0.25, "normal", 102),
    "gqa_b2_m256_n32768": GqaConfig("gqa_b2_m256_n32768", 2, 256, 32768, 0.2, "normal", 103),
    "gqa_b64_m8_n8192": GqaConfig("gqa_b64_m8_n8192", 64, 8, 8192, 0.25, "normal", 104),
    "gqa_b128_m256_n16384": GqaConfig("gqa_b128_m256_n16384", 128, 256, 16384, 0.2, "uniform", 105),
    "gqa_b64_m1_n4096_d128": GqaConfig("gqa_b64_m1_n4096_d128", 64, 1, 4096, 0.25, "normal", 106,
                                       D=128),
}
CONFIG_ORDER = list(CONFIGS)
BENCH_CONFIG = "gqa_b16_m256_n4096"


def make_qkv(B: int, M: int, N: int, *, seed: int, qk_std: float = 0.25,
             v_dist: str = "normal", D: int = HEAD_DIM):
    """Return (q, k, v) as C-contiguous numpy float16 arrays.

    q: (B, M, D), k: (B, D, N), v: (B, N, D).
    """
    if v_dist not in ("normal", "uniform"):
        raise ValueError(f"unknown v_dist {v_dist!r}")
    rng = np.random.Generator(np.random.PCG64(seed))
    q = (rng.standard_normal((B, M, D)) * qk_std).astype(np.float16)
    k = (rng.standard_normal((B, D, N)) * qk_std).astype(np.float16)
    if v_dist == "normal":
        v = rng.standard_normal((B, N, D)).astype(np.float16)
    else:
        v = rng.uniform(-1.0, 1.0, (B, N, D)).astype(np.float16)
    return np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(v)


def make_config(cfg: GqaConfig | str, seed: int | None = None):
    """Inputs for one of the named workloads (optionally with another seed)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    return make_qkv(cfg.B, cfg.M, cfg.N, seed=cfg.seed if seed is None else seed,
                    qk_std=cfg.qk_std, v_dist=cfg.v_dist, D=cfg.D)
