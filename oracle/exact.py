"""Exact-rational brute force of the block-quantized product (tiny shapes).

TEST INFRASTRUCTURE (part of the oracle; see ``oracle/__init__.py``).

Every binary16 / binary32 scale is an exact dyadic rational, so the product of
the dequantized operands, y[m,n] = sum_k deq(X)[m,k] * deq(W)[n,k], has one
exact value.  This module computes it element by element with
``fractions.Fraction`` straight from the format definitions (value =
d*sc*q - dmin*m for Q4_K, d*sc*(q-32) for Q6_K, d*q for Q8_0, Q8_K and Q8_1),
with no blocking or factoring, for shapes small enough for pure Python.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from . import ref_fp64


def _fr(x) -> Fraction:
    return Fraction(float(x))


def deq_weights_exact(wtype: int, Wq: np.ndarray, N: int, K: int):
    Wq = np.asarray(Wq, np.uint8).reshape(N, -1)
    out = [[Fraction(0)] * K for _ in range(N)]
    if wtype in (0, 5):
        if wtype == 0:
            d, dmin, sc, m, q = ref_fp64.q4k_decode_fields(Wq.reshape(N, K // 256, 144))
        else:
            d, dmin, sc, m, q = ref_fp64.q5k_decode_fields(Wq.reshape(N, K // 256, 176))
        for n in range(N):
            for b in range(K // 256):
                dd, dm = _fr(d[n, b]), _fr(dmin[n, b])
                for i in range(256):
                    j = i // 32
                    out[n][b * 256 + i] = dd * int(sc[n, b, j]) * int(q[n, b, i]) - dm * int(m[n, b, j])
    elif wtype == 1:
        d, sc, q = ref_fp64.q6k_decode_fields(Wq.reshape(N, K // 256, 210))
        for n in range(N):
            for b in range(K // 256):
                dd = _fr(d[n, b])
                for i in range(256):
                    out[n][b * 256 + i] = dd * int(sc[n, b, i // 16]) * (int(q[n, b, i]) - 32)
    else:
        blocks = Wq.reshape(N, K // 32, 34)
        for n in range(N):
            for b in range(K // 32):
                dd = _fr(np.frombuffer(blocks[n, b, 0:2].tobytes(), np.float16)[0])
                qv = blocks[n, b, 2:34].view(np.int8)
                for i in range(32):
                    out[n][b * 32 + i] = dd * int(qv[i])
    return out


def deq_act_exact(act):
    qs = act.qs
    M, K = qs.shape
    out = [[Fraction(0)] * K for _ in range(M)]
    if hasattr(act, "bsums"):
        for m in range(M):
            for k in range(K):
                out[m][k] = _fr(act.d[m, k // 256]) * int(qs[m, k])
    else:
        dv = np.asarray(act.d, np.uint16).view(np.float16)
        for m in range(M):
            for k in range(K):
                out[m][k] = _fr(dv[m, k // 32]) * int(qs[m, k])
    return out


def gemm_exact(wtype: int, Wq: np.ndarray, N: int, K: int, act):
    """Exact Y[m][n] as Fractions (list of lists)."""
    A = deq_act_exact(act)
    Wd = deq_weights_exact(wtype, Wq, N, K)
    M = len(A)
    return [[sum((A[m][k] * Wd[n][k] for k in range(K)), Fraction(0)) for n in range(N)]
            for m in range(M)]
