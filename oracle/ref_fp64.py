"""Plain definition of the block-quantized product in fp64.

TEST INFRASTRUCTURE (part of the oracle; see ``oracle/__init__.py``).

Y = deq(Xq) . deq(W)^T computed in float64 from the *quantized* operands:
the "f64 dequant band" of [P2] vllm.cpp PR #2890, commit "kROCM keep-quant
provider" (Y = X * W^T, max relative error 5e-4 against f64 dequantization).

The block layouts are decoded here with numpy, independently of vq_oracle.c:

* Q4_K (144 B): d f16 @0, dmin f16 @2, scales @4..16, nibbles @16..144.
  scales byte j<8: bits 0-5 = sc_j, bits 6-7 = bits 0-1 of m_j; byte 8+(j>>1)
  nibble (j&1) = bits 2-5 of m_j.  Byte 32c+l of the nibbles: low = element
  64c+l, high = element 64c+32+l.  value = d*sc*q - dmin*m.
* Q6_K (210 B): ql @0..128, qh @128..192, int8 sc[16] @192, d f16 @208.
  Element e (h=e//128, r=e%128): low nibble r//64 of ql[64h + r%64], bit pair
  r//32 of qh[32h + r%32].  value = d*sc[e//16]*(q-32).
* Q8_0 (34 B): d f16 @0, int8 q @2.  value = d*q.
* Q5_K (176 B): the Q4_K header @0..16, fifth-bit plane @16..48 (bit j of
  byte 16+l = bit 4 of element 32j+l), the Q4_K nibbles @48..176.
* Q8_K activation: a = d[m, i//256] * qs[m, i].
* Q8_1 activation: a = f16(d)[m, i//32] * qs[m, i].
"""
from __future__ import annotations

import numpy as np


def _f16(b: np.ndarray) -> np.ndarray:
    """Little-endian binary16 from two byte columns [..., 2] -> float64."""
    bits = b[..., 0].astype(np.uint16) | (b[..., 1].astype(np.uint16) << 8)
    return bits.view(np.float16).astype(np.float64)


def q4k_decode_fields(blocks: np.ndarray):
    """blocks uint8 [..., 144] -> d, dmin [...]; sc, m [..., 8]; q [..., 256]."""
    b = np.asarray(blocks, np.uint8)
    d = _f16(b[..., 0:2])
    dmin = _f16(b[..., 2:4])
    s = b[..., 4:16].astype(np.int64)
    j = np.arange(8)
    sc = s[..., j] & 63
    hi4 = (s[..., 8 + (j >> 1)] >> (4 * (j & 1))) & 15
    m = (s[..., j] >> 6) | (hi4 << 2)
    qs = b[..., 16:144].astype(np.int64).reshape(b.shape[:-1] + (4, 32))
    lo = qs & 15
    hi = qs >> 4
    q = np.concatenate([lo[..., :, None, :], hi[..., :, None, :]], axis=-2)  # [...,4,2,32]
    q = q.reshape(b.shape[:-1] + (256,))
    return d, dmin, sc, m, q


def q5k_decode_fields(blocks: np.ndarray):
    """blocks uint8 [..., 176] -> d, dmin [...]; sc, m [..., 8]; q [..., 256] in 0..31.
    Bytes 0..15 and 48..175 are a Q4_K block's header and nibbles; bit j of
    byte 16 + l is bit 4 of element 32j + l."""
    b = np.asarray(blocks, np.uint8)
    as_q4k = np.concatenate([b[..., 0:16], b[..., 48:176]], axis=-1)
    d, dmin, sc, m, q = q4k_decode_fields(as_q4k)
    e = np.arange(256)
    qh = b[..., 16:48].astype(np.int64)
    q = q | (((qh[..., e % 32] >> (e // 32)) & 1) << 4)
    return d, dmin, sc, m, q


def q6k_decode_fields(blocks: np.ndarray):
    """blocks uint8 [..., 210] -> d [...]; sc [..., 16] (int8); q [..., 256] in 0..63."""
    b = np.asarray(blocks, np.uint8)
    e = np.arange(256)
    h, r = e // 128, e % 128
    ql = b[..., 0:128].astype(np.int64)
    qh = b[..., 128:192].astype(np.int64)
    lo = (ql[..., 64 * h + r % 64] >> (4 * (r // 64))) & 15
    hi = (qh[..., 32 * h + r % 32] >> (2 * (r // 32))) & 3
    q = lo | (hi << 4)
    sc = b[..., 192:208].view(np.int8).astype(np.int64)
    d = _f16(b[..., 208:210])
    return d, sc, q


def dequant_weights(wtype: int, Wq: np.ndarray, N: int, K: int) -> np.ndarray:
    """Block bytes [N, row_bytes] -> fp64 [N, K]."""
    Wq = np.asarray(Wq, np.uint8).reshape(N, -1)
    if wtype == 0:
        blocks = Wq.reshape(N, K // 256, 144)
        d, dmin, sc, m, q = q4k_decode_fields(blocks)
        sub = np.arange(256) // 32
        w = d[..., None] * sc[..., sub] * q - dmin[..., None] * m[..., sub]
        return w.reshape(N, K)
    if wtype == 5:
        blocks = Wq.reshape(N, K // 256, 176)
        d, dmin, sc, m, q = q5k_decode_fields(blocks)
        sub = np.arange(256) // 32
        w = d[..., None] * sc[..., sub] * q - dmin[..., None] * m[..., sub]
        return w.reshape(N, K)
    if wtype == 1:
        blocks = Wq.reshape(N, K // 256, 210)
        d, sc, q = q6k_decode_fields(blocks)
        sub = np.arange(256) // 16
        w = d[..., None] * sc[..., sub] * (q - 32)
        return w.reshape(N, K)
    blocks = Wq.reshape(N, K // 32, 34)
    d = _f16(blocks[..., 0:2])
    q = blocks[..., 2:34].view(np.int8).astype(np.float64)
    return (d[..., None] * q).reshape(N, K)


def dequant_q8k(qs: np.ndarray, d: np.ndarray) -> np.ndarray:
    M, K = qs.shape
    return (d.astype(np.float64)[:, :, None] * qs.reshape(M, K // 256, 256)).reshape(M, K)


def dequant_q8_1(qs: np.ndarray, d_bits: np.ndarray) -> np.ndarray:
    M, K = qs.shape
    d = np.asarray(d_bits, np.uint16).view(np.float16).astype(np.float64)
    return (d[:, :, None] * qs.reshape(M, K // 32, 32)).reshape(M, K)


def dequant_act(act) -> np.ndarray:
    if hasattr(act, "bsums"):
        return dequant_q8k(act.qs, act.d)
    return dequant_q8_1(act.qs, act.d)


def gemm_fp64(wtype: int, Wq: np.ndarray, N: int, K: int, act) -> np.ndarray:
    """Y64 = deq(Xq) @ deq(W)^T in float64."""
    A = dequant_act(act)
    Wd = dequant_weights(wtype, Wq, N, K)
    return A @ Wd.T


def max_rel_err(y: np.ndarray, ref: np.ndarray, floor_frac: float = 1e-2):
    """max_i |y_i - r_i| / max(|r_i|, floor_frac * rms(r)) and the unfloored max."""
    y = np.asarray(y, np.float64)
    r = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    den = np.maximum(np.abs(r), floor_frac * rms)
    den = np.where(den == 0, 1.0, den)
    err = np.abs(y - r)
    floored = float(np.max(err / den)) if r.size else 0.0
    raw_den = np.where(np.abs(r) == 0, 1.0, np.abs(r))
    unfloored = float(np.max(err / raw_den)) if r.size else 0.0
    return floored, unfloored


def nmse(y: np.ndarray, ref: np.ndarray) -> float:
    """sum (y - o)^2 / sum o^2 over one call's whole output."""
    y = np.asarray(y, np.float64)
    o = np.asarray(ref, np.float64)
    den = float(np.sum(o * o))
    num = float(np.sum((y - o) ** 2))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den
