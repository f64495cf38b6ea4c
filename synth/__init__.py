"""Seeded synthetic inputs for the DeepSeekMoE layer forward.

This module only draws numbers: it holds none of the layer's arithmetic (no
quantisation, routing, GEMM or combine). Both the CPU oracle and the GPU path
take their inputs from here, so that the two are compared on identical values.

Workload presets follow the DeepSeek-V3 MoE configuration printed on the
lpnh.cn reproduction guide ("从技术报告到可跑配置", section 3, the model JSON:
256 routed experts, 1 shared, 8 per token, intermediate 2048,
routed_scaling_factor 2.5, expert_bias_update_rate 0.001) and the hidden size
7168 given in the same section's MLA JSON. The node/group limit (tokens reach at
most 4 groups, a group scored by the sum of its highest affinities) follows the
2kiu.com DeepSeek-V3 report digest, section 3.4.

Generation recipe (one PCG64 stream per tensor, from SeedSequence(seed).spawn in a
fixed order: x, router weight, bias, shared experts, routed experts):
  * x: N(0,1) float32, rounded to bfloat16 (RNE) unless the preset keeps fp32;
  * router weight [N_r, H]: N(0, 1/H) float32;
  * bias [N_r]: zeros or U(-0.01, 0.01) per preset, float32;
  * expert weights W1, W3 [I, H] with N(0, 1/H) and W2 [H, I] with N(0, 1/I),
    float32 (quantised to E4M3 128x128 blocks by whoever consumes them);
  * skewed preset: tokens drawn from 64 Gaussian clusters with Zipf(1.1)
    frequencies, centroid 2.0 * unit(router row e_j), noise N(0, I_H).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """Shapes and hyper-parameters of one MoE layer (field names after the model JSON)."""

    name: str
    tokens: int                      # T
    hidden_size: int                 # H
    num_experts: int                 # N_r, routed experts
    num_shared_experts: int          # N_s
    num_experts_per_tok: int         # k
    moe_intermediate_size: int       # I
    n_group: int = 1                 # G (1 = no group limit)
    topk_group: int = 1              # G_k groups kept per token
    group_score_topn: int = 2        # affinities summed per group score
    routed_scaling_factor: float = 2.5
    expert_bias_update_rate: float = 0.001
    x_dtype: str = "bf16"            # "fp32" or "bf16"
    bias_init: str = "zeros"         # "zeros" or "uniform0.01"
    skewed: bool = False
    seed: int = 0

    def with_tokens(self, tokens: int) -> "MoEConfig":
        return dataclasses.replace(self, tokens=tokens)


PRESETS = {
    "tiny": MoEConfig("tiny", 64, 256, 16, 1, 4, 128, x_dtype="fp32"),
    "reduced": MoEConfig("reduced", 2048, 2048, 64, 2, 6, 1024, bias_init="uniform0.01"),
    "v3_prefill": MoEConfig("v3_prefill", 4096, 7168, 256, 1, 8, 2048, n_group=8, topk_group=4),
    "v3_decode": MoEConfig("v3_decode", 128, 7168, 256, 1, 8, 2048, n_group=8, topk_group=4),
    "v3_skewed": MoEConfig("v3_skewed", 16384, 7168, 256, 1, 8, 2048, n_group=8, topk_group=4,
                           skewed=True),
}

N_CLUSTERS = 64
ZIPF_S = 1.1
CENTROID_NORM = 2.0


def _children(cfg: MoEConfig):
    n = 3 + 3 * cfg.num_shared_experts + 3 * cfg.num_experts
    return np.random.SeedSequence(cfg.seed).spawn(n)


def _rng(ss) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(ss))


def to_bf16_exact(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (RNE) and return them as float32 (exact)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def router_weight(cfg: MoEConfig) -> np.ndarray:
    g = _rng(_children(cfg)[1])
    w = g.standard_normal((cfg.num_experts, cfg.hidden_size), dtype=np.float32)
    return (w * np.float32(1.0 / np.sqrt(cfg.hidden_size))).astype(np.float32)


def expert_bias(cfg: MoEConfig) -> np.ndarray:
    if cfg.bias_init == "zeros":
        return np.zeros(cfg.num_experts, dtype=np.float32)
    g = _rng(_children(cfg)[2])
    return g.uniform(-0.01, 0.01, cfg.num_experts).astype(np.float32)


def hidden_states(cfg: MoEConfig, step: Optional[int] = None) -> np.ndarray:
    """Token hidden states [T, H] as float32 values (bf16-exact unless x_dtype is fp32).

    ``step`` selects a fresh batch for multi-step runs (seed = step); None uses the
    preset's own stream.
    """
    ss = _children(cfg)[0] if step is None else np.random.SeedSequence([cfg.seed, 1_000_003, step])
    g = _rng(ss)
    if not cfg.skewed:
        x = g.standard_normal((cfg.tokens, cfg.hidden_size), dtype=np.float32)
    else:
        wr = router_weight(cfg)
        perm = _rng(np.random.SeedSequence([cfg.seed, 77])).permutation(cfg.num_experts)[:N_CLUSTERS]
        rows = wr[perm].astype(np.float64)
        cent = (CENTROID_NORM * rows / np.linalg.norm(rows, axis=1, keepdims=True)).astype(np.float32)
        p = np.arange(1, N_CLUSTERS + 1, dtype=np.float64) ** (-ZIPF_S)
        p /= p.sum()
        cl = g.choice(N_CLUSTERS, size=cfg.tokens, p=p)
        x = g.standard_normal((cfg.tokens, cfg.hidden_size), dtype=np.float32)
        x += cent[cl]
    if cfg.x_dtype == "bf16":
        x = to_bf16_exact(x)
    return np.ascontiguousarray(x, dtype=np.float32)


def _expert_triplet(cfg: MoEConfig, base: int):
    ch = _children(cfg)
    H, I = cfg.hidden_size, cfg.moe_intermediate_size
    sh = np.float32(1.0 / np.sqrt(H))
    si = np.float32(1.0 / np.sqrt(I))
    w1 = _rng(ch[base]).standard_normal((I, H), dtype=np.float32)
    w1 *= sh
    w3 = _rng(ch[base + 1]).standard_normal((I, H), dtype=np.float32)
    w3 *= sh
    w2 = _rng(ch[base + 2]).standard_normal((H, I), dtype=np.float32)
    w2 *= si
    return w1, w3, w2


def shared_expert_weights(cfg: MoEConfig, s: int):
    """(W1 [I,H], W3 [I,H], W2 [H,I]) float32 of shared expert s."""
    assert 0 <= s < cfg.num_shared_experts
    return _expert_triplet(cfg, 3 + 3 * s)


def routed_expert_weights(cfg: MoEConfig, e: int):
    """(W1 [I,H], W3 [I,H], W2 [H,I]) float32 of routed expert e."""
    assert 0 <= e < cfg.num_experts
    return _expert_triplet(cfg, 3 + 3 * cfg.num_shared_experts + 3 * e)


def map_experts(cfg: MoEConfig, fn, experts, shared: bool = False, threads: Optional[int] = None):
    """Generate the weights of many experts on a thread pool and call fn(e, (w1, w3, w2)).

    Results of fn are returned in the order of ``experts``. Generation releases the GIL.
    """
    gen = shared_expert_weights if shared else routed_expert_weights
    threads = threads or min(16, os.cpu_count() or 1)
    experts = list(experts)
    out = [None] * len(experts)
    with ThreadPoolExecutor(threads) as ex:
        futs = {i: ex.submit(gen, cfg, e) for i, e in enumerate(experts[:threads])}
        nxt = len(futs)
        for i in range(len(experts)):
            w = futs.pop(i).result()
            if nxt < len(experts):
                futs[nxt] = ex.submit(gen, cfg, experts[nxt])
                nxt += 1
            out[i] = fn(experts[i], w)
    return out
