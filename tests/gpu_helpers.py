"""Helpers for the GPU parity tests: moving arrays, reading the planar
activation bytes back, and printing the case before each GPU step."""
import sys

import numpy as np

import block_quantized_matmul_fp32_amd as vq
import oracle


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def planes_q8k(buf: np.ndarray, M: int, K: int):
    """(qs int8 [M,K], d fp32 [M,K/256], bsums int16 [M,K/16]) from a planar Q8_K buffer."""
    od = vq.act_d_offset(vq.Q8_K, M, K)
    oa = vq.act_aux_offset(vq.Q8_K, M, K)
    qs = buf[: M * K].view(np.int8).reshape(M, K)
    d = buf[od: od + M * (K // 256) * 4].view(np.float32).reshape(M, K // 256)
    bs = buf[oa: oa + M * (K // 16) * 2].view(np.int16).reshape(M, K // 16)
    return qs, d, bs


def planes_q8_1(buf: np.ndarray, M: int, K: int):
    od = vq.act_d_offset(vq.Q8_1, M, K)
    oa = vq.act_aux_offset(vq.Q8_1, M, K)
    qs = buf[: M * K].view(np.int8).reshape(M, K)
    d = buf[od: od + M * (K // 32) * 2].view(np.uint16).reshape(M, K // 32)
    s = buf[oa: oa + M * (K // 32) * 2].view(np.uint16).reshape(M, K // 32)
    return qs, d, s


def pack_act(act, wtype):
    """Planar buffer bytes (numpy uint8) of an oracle activation object."""
    if wtype == oracle.Q8_0:
        M, K = act.qs.shape
        buf = np.zeros(vq.act_bytes(vq.Q8_1, M, K), np.uint8)
        od = vq.act_d_offset(vq.Q8_1, M, K)
        oa = vq.act_aux_offset(vq.Q8_1, M, K)
        buf[: M * K] = act.qs.reshape(-1).view(np.uint8)
        buf[od: od + act.d.nbytes] = act.d.reshape(-1).view(np.uint8)
        buf[oa: oa + act.s.nbytes] = act.s.reshape(-1).view(np.uint8)
        return buf
    M, K = act.qs.shape
    buf = np.zeros(vq.act_bytes(vq.Q8_K, M, K), np.uint8)
    od = vq.act_d_offset(vq.Q8_K, M, K)
    oa = vq.act_aux_offset(vq.Q8_K, M, K)
    buf[: M * K] = act.qs.reshape(-1).view(np.uint8)
    buf[od: od + act.d.nbytes] = act.d.reshape(-1).view(np.uint8)
    buf[oa: oa + act.bsums.nbytes] = act.bsums.reshape(-1).view(np.uint8)
    return buf


# The GEMM's fp32 tolerance: NMSE against the oracle's binary32 outputs and
# relative error (floored at 1% of the rms) against the fp64 dequantized product.
NMSE_MAX = 1e-6
REL_MAX = 5e-4


def fp64_cells(wtype, Wq, N, K, act, ms, ns):
    """fp64 dequantized product deq(x_m) . deq(w_n) at the cells (ms[i], ns[i]),
    dequantizing only the rows the cells touch."""
    from oracle import ref_fp64
    ms = np.asarray(ms, np.int64)
    ns = np.asarray(ns, np.int64)
    um, im = np.unique(ms, return_inverse=True)
    un, jn = np.unique(ns, return_inverse=True)
    Wrows = np.asarray(Wq, np.uint8).reshape(N, -1)[un]
    Wd = ref_fp64.dequant_weights(wtype, Wrows, un.size, K)
    if hasattr(act, "bsums"):
        A = ref_fp64.dequant_q8k(act.qs[um], act.d[um])
    else:
        A = ref_fp64.dequant_q8_1(act.qs[um], act.d[um])
    return np.einsum("ik,ik->i", A[im], Wd[jn])


def assert_close(got, ref, what, r64=None):
    """Every value finite, NMSE(got, ref) <= 1e-6 and max relative error <= 5e-4
    against r64 (the fp64 product) -- or against ref itself when r64 is not given."""
    from oracle import ref_fp64
    got = np.asarray(got, np.float32)
    assert np.isfinite(got).all(), "%s: non-finite outputs" % what
    e = ref_fp64.nmse(got, ref)
    assert e <= NMSE_MAX, "%s: NMSE %.3g > %.1g" % (what, e, NMSE_MAX)
    rel = ref_fp64.max_rel_err(got, ref if r64 is None else r64)[0]
    assert rel <= REL_MAX, "%s: max relative error %.3g > %.1g" % (what, rel, REL_MAX)


# Weight types whose MFMA GEMM keeps the oracle's fixed-order binary32 combine
# (bit-identical outputs); the K-quant GEMMs are held to the tolerance above.
EXACT_GEMM = {oracle.Q8_0}


def assert_gemm(wtype, got, ref, what, r64=None):
    if wtype in EXACT_GEMM:
        assert_bitwise(got, ref, what)
    else:
        assert_close(got, ref, what, r64)


def bits(a):
    a = np.ascontiguousarray(a, np.float32)
    return a.view(np.uint32)


def assert_bitwise(got, ref, what):
    g, r = bits(got), bits(ref)
    bad = np.nonzero(g.reshape(-1) != r.reshape(-1))[0]
    assert bad.size == 0, "%s: %d of %d differ; first at %d: got %r want %r" % (
        what, bad.size, g.size, bad[0], got.reshape(-1)[bad[0]], ref.reshape(-1)[bad[0]])
