"""Seeded synthetic inputs for the SharQ linear layer.

This module only draws random numbers and rounds them to bf16: it holds none of
the layer's arithmetic (no normalisation, masking, quantisation or products).
Both the CPU oracle and the HIP path take their inputs from here.

Workloads (the pages evaluate on real model activations; these synthetic laws
stand in for them, with the layer shapes of the models the SharQ abstract
names, Llama-3.1-8B and Qwen3-30B-A3B):

* ``tiny``   X[16,256] ~ N(0,1), channels {3,77,130,201} scaled by 40,
             gamma ~ U(0.8,1.2), W[256,256] ~ N(0,0.02).
* ``qkv``    X[2048,4096] ~ N(0,1) with max(1, round(0.002 K)) outlier channels
             scaled by log-uniform factors in [20,100]; gamma; W[6144,4096].
* ``gateup`` as ``qkv`` with W[28672,4096].
* ``down``   X = bf16(SiLU(G) * U), G,U ~ N(0,1) [2048,14336]; no gamma;
             W[4096,14336].
* ``decode`` X[M,4096] (M in {1,8,32,64}) with the ``qkv`` law; no gamma;
             W[4096,4096].
* ``moe``    128 experts, top-8 of 4096 tokens under a seeded Zipf(1.1) router.

Random source: ``numpy.random.Generator(PCG64(seed))``.  Draw order inside one
activation: outlier channel set, outlier factors, X; then gamma, then W.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_from_f32",
    "f32_from_bf16_bits",
    "outlier_activations",
    "silu_product_activations",
    "norm_weight",
    "linear_weight",
    "layer_inputs",
    "zipf_router",
    "moe_inputs",
    "CONFIGS",
]


def bf16_bits_from_f32(a) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def f32_from_bf16_bits(b) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def outlier_activations(rng, M: int, K: int, channels=None, factor=None,
                        frac: float = 0.002, lo: float = 20.0, hi: float = 100.0) -> np.ndarray:
    """N(0,1) activations with a few outlier channels; bf16 bits [M,K].

    ``channels``/``factor`` fix the outlier set (the tiny workload); otherwise
    max(1, round(frac*K)) channels are drawn without replacement and scaled by
    log-uniform factors in [lo, hi].
    """
    if channels is None:
        n = max(1, int(round(frac * K)))
        channels = rng.choice(K, n, replace=False)
        scale = np.exp(rng.uniform(np.log(lo), np.log(hi), n)).astype(np.float32)
    else:
        channels = np.asarray(channels)
        scale = np.full(len(channels), factor, dtype=np.float32)
    x = rng.standard_normal((M, K), dtype=np.float32)
    x[:, channels] *= scale
    return bf16_bits_from_f32(x)


def silu_product_activations(rng, M: int, K: int) -> np.ndarray:
    """bf16(SiLU(G) * U) with G, U ~ N(0,1): heavy-tailed MLP down-projection inputs."""
    g = rng.standard_normal((M, K), dtype=np.float32)
    u = rng.standard_normal((M, K), dtype=np.float32)
    return bf16_bits_from_f32(g / (np.float32(1) + np.exp(-g)) * u)


def norm_weight(rng, K: int) -> np.ndarray:
    return bf16_bits_from_f32(rng.uniform(0.8, 1.2, K).astype(np.float32))


def linear_weight(rng, N: int, K: int, std: float = 0.02) -> np.ndarray:
    """nn.Linear-oriented weight [N(out), K(in)] ~ N(0, std), bf16 bits."""
    return bf16_bits_from_f32(rng.standard_normal((N, K), dtype=np.float32) * np.float32(std))


# name -> (M, K, N, law, rmsnorm)
CONFIGS = {
    "tiny": (16, 256, 256, "tiny", True),
    "qkv": (2048, 4096, 6144, "outlier", True),
    "gateup": (2048, 4096, 28672, "outlier", True),
    "down": (2048, 14336, 4096, "silu", False),
    "decode1": (1, 4096, 4096, "outlier", False),
    "decode8": (8, 4096, 4096, "outlier", False),
    "decode32": (32, 4096, 4096, "outlier", False),
    "decode64": (64, 4096, 4096, "outlier", False),
}


def layer_inputs(name: str, seed: int = 0, M: int | None = None, with_weight: bool = True):
    """Inputs of one workload: dict(x, gamma|None, w, eps, M, K, N).

    ``M`` overrides the row count (same law, same K/N) for reduced-size cases.
    """
    M0, K, N, law, norm = CONFIGS[name]
    M = M0 if M is None else M
    rng = _rng(seed)
    if law == "tiny":
        x = outlier_activations(rng, M, K, channels=[3, 77, 130, 201], factor=40.0)
    elif law == "outlier":
        x = outlier_activations(rng, M, K)
    elif law == "silu":
        x = silu_product_activations(rng, M, K)
    else:
        raise ValueError(law)
    gamma = norm_weight(rng, K) if norm else None
    w = linear_weight(rng, N, K) if with_weight else None
    return dict(x=x, gamma=gamma, w=w, eps=1e-5, M=M, K=K, N=N)


def zipf_router(rng, tokens: int = 4096, experts: int = 128, top_k: int = 8, s: float = 1.1):
    """Seeded top-k routing with Zipf(s) expert popularity.

    A random permutation ranks the experts; expert e is drawn with probability
    proportional to (1 + rank(e))^-s.  Each token draws ``top_k`` distinct
    experts without replacement.  Returns (expert_of_row, token_of_row,
    seg_offsets) with rows sorted stably by (expert, token).
    """
    rank = rng.permutation(experts)
    p = (1.0 + rank) ** (-s)
    p = p / p.sum()
    choice = np.empty((tokens, top_k), dtype=np.int64)
    for t in range(tokens):
        choice[t] = rng.choice(experts, top_k, replace=False, p=p)
    expert = choice.reshape(-1)
    token = np.repeat(np.arange(tokens, dtype=np.int64), top_k)
    order = np.lexsort((token, expert))
    expert, token = expert[order], token[order]
    seg = np.zeros(experts + 1, dtype=np.int64)
    np.add.at(seg, expert + 1, 1)
    seg = np.cumsum(seg)
    return expert.astype(np.int32), token.astype(np.int32), seg


def moe_inputs(seed: int = 0, tokens: int = 4096, experts: int = 128, top_k: int = 8,
               d_model: int = 2048, d_ff: int = 768, with_weights: bool = True):
    """Qwen3-30B-A3B-shaped expert layer inputs.

    gate/up: X_tok[tokens, d_model]; per expert W_gu[2*d_ff, d_model].
    down:    X_down[tokens*top_k, d_ff] (expert-sorted rows, an independent
             draw with the same outlier law); per expert W_d[d_model, d_ff].
    No RMSNorm in either.
    """
    rng = _rng(seed)
    expert, token, seg = zipf_router(rng, tokens, experts, top_k)
    x_tok = outlier_activations(rng, tokens, d_model)
    x_down = outlier_activations(rng, tokens * top_k, d_ff)
    w_gu = w_d = None
    if with_weights:
        w_gu = np.stack([linear_weight(rng, 2 * d_ff, d_model) for _ in range(experts)])
        w_d = np.stack([linear_weight(rng, d_model, d_ff) for _ in range(experts)])
    return dict(expert=expert, token=token, seg=seg, x_tok=x_tok, x_down=x_down,
                w_gu=w_gu, w_d=w_d, tokens=tokens, experts=experts, top_k=top_k,
                d_model=d_model, d_ff=d_ff)
