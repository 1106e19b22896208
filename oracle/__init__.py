"""CPU oracle for the block-quantized matmul.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package.  It shares no code with
the HIP library (``block_quantized_matmul_fp32_amd``) and never imports it.

Three independent layers:

* ``vq_oracle.c`` (loaded here through ctypes): the plain binary32 oracle --
  weight encoders, the Q8_K / Q8_1 activation quantizers, the integer block
  dots in the fixed accumulation order, routing and the weighted expert sum.
* ``ref_fp64``: the plain definition of the product, dequantize-then-matmul in
  fp64, with its own numpy decoding of the block layouts.
* ``exact``: brute force in exact rationals for tiny shapes.

Pages cited in docstrings:
  [P2] vllm.cpp PR #2890 "fuse silu-mul with Q8_K quant epilogue"
  [P3] strix-llama.cpp PR #18 "Optimize ROCM Prefill and Decode"
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

Q4_K, Q6_K, Q8_0, Q5_K = 0, 1, 2, 5
WEIGHT_TYPES = {"Q4_K": Q4_K, "Q6_K": Q6_K, "Q8_0": Q8_0}
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210, Q8_0: 34, Q5_K: 176}
BLOCK_ELEMS = {Q4_K: 256, Q6_K: 256, Q8_0: 32, Q5_K: 256}

_lib = None


def build(force: bool = True) -> str:
    """Compile vq_oracle.c with gcc (no FMA contraction, no fast math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(path):
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
    L.oracle_f32_to_f16.restype = ctypes.c_uint16
    L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    L.oracle_f16_to_f32.restype = ctypes.c_float
    L.oracle_q4k_fields.argtypes = [P, P, P, P, P]
    L.oracle_q6k_fields.argtypes = [P, P, P, P]
    L.oracle_q4k_build.argtypes = [ctypes.c_uint16, ctypes.c_uint16, P, P, P, P]
    L.oracle_q5k_fields.argtypes = [P, P, P, P, P]
    L.oracle_q5k_build.argtypes = [ctypes.c_uint16, ctypes.c_uint16, P, P, P, P]
    L.oracle_q6k_build.argtypes = [ctypes.c_uint16, P, P, P]
    L.oracle_quantize_weights.argtypes = [ctypes.c_int, P, I64, I64, P]
    L.oracle_quantize_q8k.argtypes = [P, I64, I64, I64, P, P, P]
    L.oracle_quantize_q8_1.argtypes = [P, I64, I64, I64, P, P, P]
    L.oracle_gemm.argtypes = [ctypes.c_int, P, I64, I64, P, P, P, I64, P, I64, ctypes.c_int]
    L.oracle_gemm_sampled.argtypes = [ctypes.c_int, P, I64, I64, P, P, P, P, P, I64, P,
                                      ctypes.c_int]
    L.oracle_subblock_sums.argtypes = [ctypes.c_int, P, P, P]
    L.oracle_route.argtypes = [P, I64, I64, I64, P, P, P]
    L.oracle_gemm_grouped.argtypes = [ctypes.c_int, P, I64, I64, I64, P, P, P, I64, P, I64,
                                      ctypes.c_int, P, ctypes.c_int]
    L.oracle_weighted_sum.argtypes = [P, P, I64, I64, I64, P]
    L.oracle_rmsnorm.argtypes = [P, P, I64, I64, I64, ctypes.c_double, P]
    L.oracle_silu_mul.argtypes = [P, P, I64, I64, I64, P]
    L.oracle_max_threads.restype = ctypes.c_int
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _bind(_LIB_PATH)
    return _lib


def _swap_library(path):
    """Point this wrapper at another build of vq_oracle.c (used by the mutation
    tests to check that the pins reject planted mistakes); returns the old one."""
    global _lib
    old = _lib
    _lib = _bind(path) if isinstance(path, str) else path
    return old


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# --------------------------------------------------------------------------
# binary16
# --------------------------------------------------------------------------
def f32_to_f16_bits(x: float) -> int:
    return int(lib().oracle_f32_to_f16(float(x)))


def f16_bits_to_f32(h: int) -> float:
    return float(lib().oracle_f16_to_f32(int(h)))


# --------------------------------------------------------------------------
# block fields
# --------------------------------------------------------------------------
def q4k_fields(block: np.ndarray):
    """(d, dmin, sc[8], m[8], q[256]) of one 144-byte Q4_K block."""
    b = np.ascontiguousarray(block, dtype=np.uint8)
    dd = np.zeros(2, np.float32)
    sc = np.zeros(8, np.int32)
    m = np.zeros(8, np.int32)
    q = np.zeros(256, np.int32)
    lib().oracle_q4k_fields(_p(b), _p(dd), _p(sc), _p(m), _p(q))
    return float(dd[0]), float(dd[1]), sc, m, q


def q6k_fields(block: np.ndarray):
    """(d, sc[16], q[256]) of one 210-byte Q6_K block (q in 0..63)."""
    b = np.ascontiguousarray(block, dtype=np.uint8)
    d = np.zeros(1, np.float32)
    sc = np.zeros(16, np.int32)
    q = np.zeros(256, np.int32)
    lib().oracle_q6k_fields(_p(b), _p(d), _p(sc), _p(q))
    return float(d[0]), sc, q


def q5k_fields(block: np.ndarray):
    """(d, dmin, sc[8], m[8], q[256]) of one 176-byte Q5_K block."""
    b = np.ascontiguousarray(block, dtype=np.uint8)
    dd = np.zeros(2, np.float32)
    sc = np.zeros(8, np.int32)
    m = np.zeros(8, np.int32)
    q = np.zeros(256, np.int32)
    lib().oracle_q5k_fields(_p(b), _p(dd), _p(sc), _p(m), _p(q))
    return float(dd[0]), float(dd[1]), sc, m, q


def q5k_build(d16: int, dmin16: int, sc, m, q) -> np.ndarray:
    out = np.zeros(176, np.uint8)
    sc = np.ascontiguousarray(sc, np.int32)
    m = np.ascontiguousarray(m, np.int32)
    q = np.ascontiguousarray(q, np.int32)
    lib().oracle_q5k_build(d16, dmin16, _p(sc), _p(m), _p(q), _p(out))
    return out


def q4k_build(d16: int, dmin16: int, sc, m, q) -> np.ndarray:
    out = np.zeros(144, np.uint8)
    sc = np.ascontiguousarray(sc, np.int32)
    m = np.ascontiguousarray(m, np.int32)
    q = np.ascontiguousarray(q, np.int32)
    lib().oracle_q4k_build(d16, dmin16, _p(sc), _p(m), _p(q), _p(out))
    return out


def q6k_build(d16: int, sc, q) -> np.ndarray:
    out = np.zeros(210, np.uint8)
    sc = np.ascontiguousarray(sc, np.int32)
    q = np.ascontiguousarray(q, np.int32)
    lib().oracle_q6k_build(d16, _p(sc), _p(q), _p(out))
    return out


# --------------------------------------------------------------------------
# encoders and quantizers
# --------------------------------------------------------------------------
def quantize_weights(wtype: int, W: np.ndarray) -> np.ndarray:
    """fp32 W [N, K] -> uint8 blocks [N, K/QK * block_bytes]."""
    W = np.ascontiguousarray(W, np.float32)
    N, K = W.shape
    qk = BLOCK_ELEMS[wtype]
    assert K % qk == 0
    out = np.zeros((N, (K // qk) * BLOCK_BYTES[wtype]), np.uint8)
    lib().oracle_quantize_weights(wtype, _p(W), N, K, _p(out))
    return out


class Q8K:
    """Q8_K activation planes: qs int8 [M,K], d fp32 [M,K/256], bsums int16 [M,K/16]."""

    def __init__(self, qs, d, bsums):
        self.qs, self.d, self.bsums = qs, d, bsums

    @property
    def shape(self):
        return self.qs.shape


class Q81:
    """Q8_1 activation planes: qs int8 [M,K], d fp16 [M,K/32], s fp16 [M,K/32]
    (the fp16 planes are held as uint16 bit patterns)."""

    def __init__(self, qs, d, s):
        self.qs, self.d, self.s = qs, d, s

    @property
    def shape(self):
        return self.qs.shape


def quantize_q8k(X: np.ndarray) -> Q8K:
    """[P2] QuantizeQ8KKWarpCoop semantics (see vq_oracle.c)."""
    X = np.ascontiguousarray(X, np.float32)
    if X.ndim == 1:
        X = X[None, :]
    M, K = X.shape
    assert K % 256 == 0
    qs = np.zeros((M, K), np.int8)
    d = np.zeros((M, K // 256), np.float32)
    bs = np.zeros((M, K // 16), np.int16)
    lib().oracle_quantize_q8k(_p(X), M, K, K, _p(qs), _p(d), _p(bs))
    return Q8K(qs, d, bs)


def quantize_q8_1(X: np.ndarray) -> Q81:
    """[P3] mul_mat_vec_q_fq quantization semantics (see vq_oracle.c)."""
    X = np.ascontiguousarray(X, np.float32)
    if X.ndim == 1:
        X = X[None, :]
    M, K = X.shape
    assert K % 32 == 0
    qs = np.zeros((M, K), np.int8)
    d = np.zeros((M, K // 32), np.uint16)
    s = np.zeros((M, K // 32), np.uint16)
    lib().oracle_quantize_q8_1(_p(X), M, K, K, _p(qs), _p(d), _p(s))
    return Q81(qs, d, s)


# --------------------------------------------------------------------------
# matmul
# --------------------------------------------------------------------------
def _act_args(wtype, act):
    if wtype == Q8_0:
        assert isinstance(act, Q81), "Q8_0 weights pair with Q8_1 activations"
        return act.qs, act.d, np.zeros(1, np.int16)
    assert isinstance(act, Q8K), "K-quant weights pair with Q8_K activations"
    return act.qs, act.d, act.bsums


def gemm(wtype: int, Wq: np.ndarray, N: int, K: int, act, nthreads: int = 1) -> np.ndarray:
    """Y[m, n] = sum_b c_b (binary32, blocks ascending) -- [P2] Y = X * W^T."""
    qs, d, bs = _act_args(wtype, act)
    M = qs.shape[0]
    Wq = np.ascontiguousarray(Wq, np.uint8)
    Y = np.zeros((M, N), np.float32)
    lib().oracle_gemm(wtype, _p(Wq), N, K, _p(qs), _p(d), _p(bs), M, _p(Y), N, int(nthreads))
    return Y


def gemm_sampled(wtype, Wq, N, K, act, ms, ns, nthreads: int = 1) -> np.ndarray:
    qs, d, bs = _act_args(wtype, act)
    ms = np.ascontiguousarray(ms, np.int64)
    ns = np.ascontiguousarray(ns, np.int64)
    out = np.zeros(ms.shape[0], np.float32)
    Wq = np.ascontiguousarray(Wq, np.uint8)
    lib().oracle_gemm_sampled(wtype, _p(Wq), N, K, _p(qs), _p(d), _p(bs), _p(ms), _p(ns),
                              ms.shape[0], _p(out), int(nthreads))
    return out


def subblock_sums(wtype: int, wblock: np.ndarray, a: np.ndarray) -> np.ndarray:
    n = {Q4_K: 8, Q6_K: 16, Q8_0: 1, Q5_K: 8}[wtype]
    out = np.zeros(n, np.int32)
    wb = np.ascontiguousarray(wblock, np.uint8)
    aa = np.ascontiguousarray(a, np.int8)
    lib().oracle_subblock_sums(wtype, _p(wb), _p(aa), _p(out))
    return out


def route(ids: np.ndarray, E: int):
    """[P3] routed-compact: counts [E], offsets [E+1], list [T*top_k]."""
    ids = np.ascontiguousarray(ids, np.int32)
    T, top_k = ids.shape
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    lst = np.zeros(T * top_k, np.int32)
    lib().oracle_route(_p(ids), T, top_k, E, _p(counts), _p(offsets), _p(lst))
    return counts, offsets, lst


def gemm_grouped(wtype, Wq, E, N, K, act, ids, nthreads: int = 1, per_row: bool = False) -> np.ndarray:
    """Y[t, s, :] = W_{ids[t,s]} . x, with x the token's row x_t (broadcast arm)
    or the pair's own row x_{t*top_k+s} (per-row arm)."""
    ids = np.ascontiguousarray(ids, np.int32)
    T, top_k = ids.shape
    qs, d, bs = _act_args(wtype, act)
    assert qs.shape[0] == (T * top_k if per_row else T), "activation rows"
    Y = np.zeros((T, top_k, N), np.float32)
    Wq = np.ascontiguousarray(Wq, np.uint8)
    lib().oracle_gemm_grouped(wtype, _p(Wq), E, N, K, _p(qs), _p(d), _p(bs), T,
                              _p(ids), top_k, int(per_row), _p(Y), int(nthreads))
    return Y


def weighted_sum(Y: np.ndarray, w: np.ndarray) -> np.ndarray:
    """[P3] weighted expert sum: slots ascending, mul then add, no FMA."""
    Y = np.ascontiguousarray(Y, np.float32)
    w = np.ascontiguousarray(w, np.float32)
    T, top_k, N = Y.shape
    out = np.zeros((T, N), np.float32)
    lib().oracle_weighted_sum(_p(Y), _p(w), T, top_k, N, _p(out))
    return out


def rmsnorm(X: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """[P2] norm-quant epilogue's producer: RMSNorm of each row, float64
    y = x / sqrt(mean(x^2) + eps) * gamma from binary32 X [M, K], gamma [K]."""
    X = np.ascontiguousarray(np.atleast_2d(X), np.float32)
    gamma = np.ascontiguousarray(gamma, np.float32)
    M, K = X.shape
    assert gamma.shape == (K,)
    out = np.zeros((M, K), np.float64)
    lib().oracle_rmsnorm(_p(X), _p(gamma), M, K, K, float(eps), _p(out))
    return out


def silu_mul(G: np.ndarray, U: np.ndarray) -> np.ndarray:
    """[P2] silu-mul quant epilogue's producer, float64
    y = g / (1 + exp(-g)) * u from binary32 G, U [M, K]."""
    G = np.ascontiguousarray(np.atleast_2d(G), np.float32)
    U = np.ascontiguousarray(np.atleast_2d(U), np.float32)
    assert G.shape == U.shape
    M, K = G.shape
    out = np.zeros((M, K), np.float64)
    lib().oracle_silu_mul(_p(G), _p(U), M, K, K, _p(out))
    return out


def max_threads() -> int:
    return int(lib().oracle_max_threads())
