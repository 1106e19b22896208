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


def bits(a):
    a = np.ascontiguousarray(a, np.float32)
    return a.view(np.uint32)


def assert_bitwise(got, ref, what):
    g, r = bits(got), bits(ref)
    bad = np.nonzero(g.reshape(-1) != r.reshape(-1))[0]
    assert bad.size == 0, "%s: %d of %d differ; first at %d: got %r want %r" % (
        what, bad.size, g.size, bad[0], got.reshape(-1)[bad[0]], ref.reshape(-1)[bad[0]])
