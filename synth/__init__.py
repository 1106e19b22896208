"""Seeded synthetic inputs for the block-quantized matmul workloads.

This module only draws random numbers: it holds none of the quantized-matmul
arithmetic (no quantizer, no block layout, no dot product).  Both the CPU
oracle side and the HIP side take their fp32 inputs from here.

Generator: numpy ``default_rng`` (PCG64) draws float64 standard normals, which
are scaled and then cast to float32.  Shapes follow the pages' Qwen-class
workloads: hidden size 2560 and intermediate size 9728 (decode K=2560), and
256 experts, top-8, 2048 tokens, experts of [512, 2048] for the routed path.
"""
from __future__ import annotations

import numpy as np

# Workloads: name -> description of the fp32 tensors (shape, seed, sigma).
WORKLOADS = {
    "tiny_q4k_gemm": {
        "desc": "Q4_K GEMM Y[8,256] = X[8,1024] . W[256,1024]^T",
        "W": ((256, 1024), 11, 0.02), "X": ((8, 1024), 12, 1.0),
    },
    "decode_gemv": {
        "desc": "M=1 GEMV: Q4_K [9728,2560] and Q6_K [2560,9728], Q8_K activations",
        "Wa": ((9728, 2560), 21, 0.02), "Wb": ((2560, 9728), 22, 0.02),
        "xa": ((2560,), 23, 1.0), "xb": ((9728,), 24, 1.0),
    },
    "prefill_gemm": {
        "desc": "M in {512, 2048}: Q4_K gate/up [9728,2560], Q6_K down [2560,9728], Q8_K activations",
        "Wgate": ((9728, 2560), 31, 0.02), "Wup": ((9728, 2560), 32, 0.02),
        "Wdown": ((2560, 9728), 33, 0.02),
        "Xh": ((2048, 2560), 34, 1.0), "Xi": ((2048, 9728), 35, 1.0),
        "outlier_seed": 36, "outlier_frac": 0.01, "outlier_scale": 20.0,
    },
    "q8_0_gemm": {
        "desc": "Q8_0 [4096,2048] x Q8_1 activations, M=2048 GEMM and M=1 GEMV on row 0",
        "W": ((4096, 2048), 41, 0.02), "X": ((2048, 2048), 42, 1.0),
    },
    "grouped_moe": {
        "desc": "256 experts Q4_K [512,2048], 2048 tokens, top-8 routing, Q8_K activations",
        "E": 256, "N": 512, "K": 2048, "T": 2048, "top_k": 8,
        "W_seed": 51, "W_sigma": 0.02, "X": ((2048, 2048), 52, 1.0),
        "ids_seed": 53, "logits_seed": 54,
    },
    "q5k_decode": {
        "desc": "Q5_K [8192,2560] decode GEMV (the GDN qkv projection shape the pages keep in Q5_K)",
        "W": ((8192, 2560), 81, 0.02), "x": ((2560,), 82, 1.0), "X": ((16, 2560), 83, 1.0),
    },
    "grouped_moe_down": {
        "desc": "per-row arm: 256 experts Q4_K [2048,512], one Q8_K row per (token, slot): "
                "[2048*8, 512], the grouped_moe routing",
        "E": 256, "N": 2048, "K": 512, "T": 2048, "top_k": 8,
        "W_seed": 61, "W_sigma": 0.02, "X": ((2048 * 8, 512), 62, 1.0),
    },
}


def normal(seed, shape, sigma: float = 1.0) -> np.ndarray:
    """float32 draw of sigma * N(0,1) from default_rng(seed) (float64 then cast)."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape) * sigma).astype(np.float32)


def tensor(workload: str, name: str) -> np.ndarray:
    shape, seed, sigma = WORKLOADS[workload][name]
    return normal(seed, shape, sigma)


def outlier_columns(K: int, seed: int = 36, frac: float = 0.01) -> np.ndarray:
    """round(frac*K) column indices from a seeded permutation (shared by all rows)."""
    rng = np.random.default_rng((seed, K))
    return np.sort(rng.permutation(K)[: int(round(frac * K))])


def prefill_activations(name: str, M: int) -> np.ndarray:
    """Xh [M,2560] or Xi [M,9728]: the first M rows of the 2048-row draw, with the
    outlier columns scaled by 20."""
    w = WORKLOADS["prefill_gemm"]
    X = tensor("prefill_gemm", name)[:M].copy()
    cols = outlier_columns(X.shape[1], w["outlier_seed"], w["outlier_frac"])
    X[:, cols] *= np.float32(w["outlier_scale"])
    return X


def expert_weights(e: int, N: int = 512, K: int = 2048, seed: int = 51,
                   sigma: float = 0.02) -> np.ndarray:
    """fp32 weights of expert e, drawn from default_rng((seed, e)) so that experts
    can be generated one at a time."""
    return normal((seed, e), (N, K), sigma)


def routing(T: int = 2048, E: int = 256, top_k: int = 8, ids_seed: int = 53,
            logits_seed: int = 54):
    """ids int32 [T, top_k]: top_k distinct experts per token, uniform; weights
    fp32 [T, top_k]: softmax over the token's own top_k N(0,1) logits (fp64)."""
    rng = np.random.default_rng(ids_seed)
    keys = rng.random((T, E))
    ids = np.argsort(keys, axis=1, kind="stable")[:, :top_k].astype(np.int32)
    logits = np.random.default_rng(logits_seed).standard_normal((T, top_k))
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


def random_ids(seed, T: int, E: int, top_k: int) -> np.ndarray:
    """Distinct uniform expert ids per token (small parity cases)."""
    rng = np.random.default_rng(seed)
    keys = rng.random((T, E))
    return np.argsort(keys, axis=1, kind="stable")[:, :top_k].astype(np.int32)


def skewed_ids(seed, T: int, E: int, top_k: int, counts_hint) -> np.ndarray:
    """Ids whose per-expert row counts follow a given pattern as closely as the
    distinct-per-token rule allows (edge cases: empty, single, full experts).
    counts_hint[e] is a sampling weight; zero weight means the expert is never used."""
    rng = np.random.default_rng(seed)
    p = np.asarray(counts_hint, np.float64)
    p = p / p.sum()
    ids = np.zeros((T, top_k), np.int32)
    for t in range(T):
        ids[t] = rng.choice(E, size=top_k, replace=False, p=p)
    return ids
