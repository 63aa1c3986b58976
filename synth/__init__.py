"""Seeded synthetic inputs for the fine-grained quantized linear layer Y = X.W.

This module is shared by both sides of every parity test and by the bench: the
CPU oracle and the HIP path receive the very same float32 arrays from here. It
only draws numbers (normals, permutations, Bernoulli masks) and applies the
outlier structure of the workloads; it holds none of the quantization
arithmetic.

Generator: numpy's Philox-4x32-10 counter-based bit generator (Salmon, Moraes,
Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011), keyed by
the pair (seed, stream) so every tensor of a workload has its own stream.

Workload shapes and distributions follow the Integer Scale summary page
("Integer Scale: A Free Lunch for Faster Fine-grained Quantization of LLMs"):
the kernel comparison of its section 5.2 (Fig. 5a, Fig. 6) uses K=4096,
N=22016; its Table 1 fixes group size 128 and amplifier 1024. The outlier
structure stands in for real LLM tensors: a few activation channels much larger
than the rest (the LLM.int8 description on the "LLMs量化算法概述" page) and a
small fraction of salient weights (the AWQ description on the same page).
No dataset or trained weights are used.
"""
from __future__ import annotations

import numpy as np

STREAM_X = 1        # activation normals
STREAM_PERM = 2     # outlier-channel permutation
STREAM_W = 3        # weight normals
STREAM_W_OUT = 4    # weight outlier Bernoulli draws
STREAM_LAYER = 10   # + layer index, for the decoder-block stack
STREAM_ROUTE = 5    # router logits of the mixture-of-experts workload
STREAM_EXPERT = 20  # + expert index, expert weights

K_LAYER = 4096
N_LAYER = 22016
GROUP = 128
ALPHA = 1024
DECODE_M = (1, 4, 16, 64, 256)
PREFILL_M = (512, 1024, 2048, 4096)

# Mixtral-8x7B experts: 8 experts per layer, 2 routed per token; the expert
# FFN linears are w1 / w3 (hidden 4096 -> 14336) and w2 (14336 -> 4096)
MIXTRAL_E = 8
MIXTRAL_TOPK = 2
MIXTRAL_HIDDEN = 4096
MIXTRAL_FFN = 14336

# LLaMA-2-7B decoder-block linears (in_features K, out_features N)
LLAMA2_7B_BLOCK = (
    ("q_proj", 4096, 4096),
    ("k_proj", 4096, 4096),
    ("v_proj", 4096, 4096),
    ("o_proj", 4096, 4096),
    ("gate_proj", 4096, 11008),
    ("up_proj", 4096, 11008),
    ("down_proj", 11008, 4096),
)


def rng(seed: int, stream: int) -> np.random.Generator:
    key = np.array([seed & 0xFFFFFFFFFFFFFFFF, stream & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key))


def normal(seed: int, stream: int, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """float32 normals N(mean, std^2), C-contiguous."""
    g = rng(seed, stream)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return np.ascontiguousarray(a)


def outlier_channels(seed: int, K: int, frac: float = 0.01) -> np.ndarray:
    """Sorted indices of round(frac*K) channels chosen by a seeded permutation."""
    n = int(round(frac * K))
    perm = rng(seed, STREAM_PERM).permutation(K)
    return np.sort(perm[:n])


def activations(seed: int, M: int, K: int, outlier_frac: float = 0.01,
                outlier_scale: float = 20.0, mean: float = 0.0, std: float = 1.0,
                relu: bool = False) -> np.ndarray:
    """X (M x K, float32): normals with whole columns (channels) scaled up.

    The outlier channels depend only on (seed, K), so the first m rows of an
    M-row draw are the m-row draw's rows too.
    """
    x = normal(seed, STREAM_X, (M, K), mean=mean, std=std)
    if outlier_frac > 0.0 and outlier_scale != 1.0:
        cols = outlier_channels(seed, K, outlier_frac)
        x[:, cols] *= np.float32(outlier_scale)
    if relu:
        np.maximum(x, np.float32(0.0), out=x)
    return x


def weights(seed: int, K: int, N: int, std: float = 0.02, outlier_prob: float = 0.0,
            outlier_scale: float = 10.0, stream: int = STREAM_W) -> np.ndarray:
    """W (K x N, float32, row-major): N(0, std^2) with optional salient elements.

    Each element is independently multiplied by outlier_scale with probability
    outlier_prob.
    """
    w = normal(seed, stream, (K, N), std=std)
    if outlier_prob > 0.0:
        u = rng(seed, stream + STREAM_W_OUT * 1000).random(size=(K, N), dtype=np.float32)
        w[u < np.float32(outlier_prob)] *= np.float32(outlier_scale)
    return w


# ---------------------------------------------------------------- workloads

def single_gemm_inputs(seed: int = 0):
    """Single layer: X 16x4096 N(0,1) with 1% channels x20; W 4096x4096 N(0,0.02)."""
    x = activations(seed, 16, 4096)
    w = weights(seed, 4096, 4096, std=0.02)
    return x, w


def layer_inputs(seed: int = 0, M: int = 256, K: int = K_LAYER, N: int = N_LAYER):
    """The K=4096, N=22016 layer: X N(0,1) + 1% channels x20, W N(0,0.02) + 0.1% x10."""
    x = activations(seed, M, K)
    w = weights(seed, K, N, std=0.02, outlier_prob=0.001, outlier_scale=10.0)
    return x, w


def w8a8_inputs(seed: int = 0, M: int = 256, K: int = 4096, N: int = 4096, relu: bool = False):
    """Asymmetric W8A8 control: X ~ N(0.5, 1) (optionally ReLU'd), W ~ N(0, 0.02)."""
    x = activations(seed, M, K, outlier_frac=0.0, mean=0.5, relu=relu)
    w = weights(seed, K, N, std=0.02)
    return x, w


def block_inputs(seed: int = 0, M: int = 1):
    """LLaMA-2-7B-shaped decoder block: one (name, X, W) per linear."""
    out = []
    for li, (name, k, n) in enumerate(LLAMA2_7B_BLOCK):
        x = activations(seed + 7919 * (li + 1), M, k)
        w = weights(seed, k, n, std=0.02, stream=STREAM_LAYER + li)
        out.append((name, x, w))
    return out


def moe_routing(seed: int, T: int, E: int = MIXTRAL_E, topk: int = MIXTRAL_TOPK,
                skew: float = 0.5):
    """Synthetic routing of T tokens to topk distinct experts each.

    Router logits are N(0,1) per (token, expert) plus a fixed per-expert bias
    N(0, skew^2), so some experts receive more tokens than others as trained
    routers do; each token takes its topk largest logits (ties broken by the
    lower expert index). Returns the (T, topk) int32 expert indices, largest
    logit first.
    """
    g = rng(seed, STREAM_ROUTE)
    bias = g.standard_normal(E) * skew
    logits = g.standard_normal((T, E)) + bias[None, :]
    order = np.argsort(-logits, axis=1, kind="stable")
    return np.ascontiguousarray(order[:, :topk].astype(np.int32))


def route_by_expert(experts: np.ndarray, E: int):
    """Sort the (token, expert) pairs by expert, tokens in order within an
    expert: returns offsets (E+1 int32, expert e's slots are offs[e] ..
    offs[e+1]-1) and the token of each slot (R = T*topk int32)."""
    T, topk = experts.shape
    flat_e = experts.reshape(-1)
    flat_t = np.repeat(np.arange(T, dtype=np.int32), topk)
    order = np.argsort(flat_e, kind="stable")
    tok = np.ascontiguousarray(flat_t[order].astype(np.int32))
    counts = np.bincount(flat_e, minlength=E)
    offs = np.zeros(E + 1, np.int32)
    offs[1:] = np.cumsum(counts)
    return offs, tok


def expert_weights(seed: int, E: int, K: int, N: int, std: float = 0.02,
                   outlier_prob: float = 0.001) -> np.ndarray:
    """(E, K, N) float32 expert weight matrices, one stream per expert."""
    return np.stack([weights(seed + 1000 * STREAM_EXPERT + e, K, N, std=std,
                             outlier_prob=outlier_prob) for e in range(E)])

