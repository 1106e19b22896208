"""GPU parity of the producers with the quantizer epilogue (needs an MI355X).

vq_rmsnorm_quant and vq_silu_mul_quant write a binary32 output Y and its
quantized blocks Xq in one launch. The bar:
  * Xq is byte-identical to the oracle's quantizer applied to the Y the
    kernel stored (and to the library's own standalone quantizer on that Y),
    with or without Y requested;
  * Y is within a relative bound of the binary64 oracle. RMSNorm over nw
    waves (min(16, ceil(steps / 4)) for many rows, 4 for up to 16 rows of at
    most 64 steps): a lane sums 4 * ceil(steps / nw) squares in order, then 4
    exchange levels, 3 adds of the row sums and nw wave partials: n =
    4 * ceil(steps / nw) + 7 + nw roundings of non-negative terms, at most n
    units of 2^-24 relative on the sum, halved by the root; the root, the
    division and the two products add at most 4 units: (n / 2 + 4) * 2^-24
    (the larger of the two layouts). SiLU-mul: 1e-6 (exp within a couple of units,
    then 1 + e, the division and the product, each correctly rounded; no
    cancellation anywhere);
  * decode: the RMSNorm bytes feed vq_gemm at M = 1 and the output is
    bit-identical to the oracle GEMM on the oracle's quantization of Y.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_helpers as H
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import block_quantized_matmul_fp32_amd as vq  # noqa: E402

TOL = {"silu": 1e-6}


def tol_rmsnorm(K):
    steps = -(-K // 256)
    n = max(4 * -(-steps // nw) + 7 + nw for nw in (4, min(16, -(-steps // 4))))
    return (n / 2 + 4) * 2.0 ** -24


def gamma_of(K, seed):
    return (1.0 + synth.normal(seed, (K,), 0.1)).astype(np.float32)


def check_bytes(act, Xq_dev, Y):
    """Xq planes == oracle quantizer on Y (the kernel's own binary32 output)."""
    M, K = Y.shape
    buf = H.host(Xq_dev)
    if act == vq.Q8_K:
        ref = oracle.quantize_q8k(Y)
        qs, d, bs = H.planes_q8k(buf, M, K)
        assert np.array_equal(qs, ref.qs)
        assert np.array_equal(d.view(np.uint32), ref.d.view(np.uint32))
        assert np.array_equal(bs, ref.bsums)
    else:
        ref = oracle.quantize_q8_1(Y)
        qs, d, s = H.planes_q8_1(buf, M, K)
        assert np.array_equal(qs, ref.qs) and np.array_equal(d, ref.d) and np.array_equal(s, ref.s)
    return ref


def planes(act, Xq_dev, M, K):
    buf = H.host(Xq_dev)
    return H.planes_q8k(buf, M, K) if act == vq.Q8_K else H.planes_q8_1(buf, M, K)


def assert_close(Y, R, tol, what):
    err = np.abs(Y.astype(np.float64) - R)
    bound = tol * np.abs(R) + 1e-30
    bad = np.nonzero(err > bound)
    assert bad[0].size == 0, "%s: %d outside %g; first at %s: got %r want %r" % (
        what, bad[0].size, tol, tuple(b[0] for b in bad), Y[tuple(b[0] for b in bad)], R[tuple(b[0] for b in bad)])


# (act, M, K, ldx, offset): aligned and strided/unaligned inputs, 1..16 steps
# per wave, a ragged last Q8_1 step, the largest K
CASES = [
    (vq.Q8_K, 5, 2560, 2560, 0),
    (vq.Q8_K, 3, 9728, 9728 + 4, 0),
    (vq.Q8_K, 2, 4096, 4096 + 3, 1),
    (vq.Q8_K, 1, 65536, 65536, 0),
    (vq.Q8_K, 2, 32768, 32768, 0),
    (vq.Q8_K, 1, 131072, 131072, 0),
    (vq.Q8_K, 40, 2560, 2560, 0),
    (vq.Q8_K, 17, 9728, 9728, 0),
    (vq.Q8_1, 4, 2080, 2080, 0),
    (vq.Q8_1, 3, 4128, 4128 + 1, 3),
    (vq.Q8_1, 2, 224, 224, 0),
    (vq.Q8_1, 33, 2080, 2080, 0),
]


def padded(X, ldx, off):
    M, K = X.shape
    Xp = np.zeros(M * ldx + off + 8, np.float32)
    view = np.lib.stride_tricks.as_strided(Xp[off:], (M, K), (4 * ldx, 4))
    view[:] = X
    return Xp


@pytest.mark.parametrize("case", range(len(CASES)))
def test_rmsnorm_quant(case):
    act, M, K, ldx, off = CASES[case]
    X = synth.normal((3200, case), (M, K))
    X[0, : min(K, 512)] *= np.float32(30.0)  # outliers that set the block scales
    g = gamma_of(K, 3201 + case)
    eps = 1e-6
    H.say("rmsnorm_quant act=%d M=%d K=%d ldx=%d off=%d" % (act, M, K, ldx, off))
    Xd = H.to_dev(padded(X, ldx, off))[off:]
    vq.reset_stats()
    Y, Xq = vq.rmsnorm_quant(act, Xd, H.to_dev(g), eps, M=M, K=K, ldx=ldx)
    Yh = H.host(Y)
    assert vq.get_stats()["rmsnorm_quant"] == 1
    assert_close(Yh, oracle.rmsnorm(X, g, eps), tol_rmsnorm(K), "rmsnorm Y")
    check_bytes(act, Xq, Yh)
    sq = vq.quantize_act(act, Y)
    for a, b in zip(planes(act, Xq, M, K), planes(act, sq, M, K)):
        assert np.array_equal(a, b), "standalone quantizer on Y"
    _, Xq2 = vq.rmsnorm_quant(act, Xd, H.to_dev(g), eps, M=M, K=K, ldx=ldx, want_y=False)
    for a, b in zip(planes(act, Xq, M, K), planes(act, Xq2, M, K)):
        assert np.array_equal(a, b), "bytes without Y"


@pytest.mark.parametrize("case", range(len(CASES)))
def test_silu_mul_quant(case):
    act, M, K, ld1, off = CASES[case]
    # gate | up interleaved per row (U = G + K, row stride 2K + pad)
    ldx = 2 * K + (ld1 - K)
    G = synth.normal((3300, case), (M, K), 3.0)
    U = synth.normal((3301, case), (M, K))
    GU = np.concatenate([G, U], axis=1)
    H.say("silu_mul_quant act=%d M=%d K=%d ldx=%d off=%d" % (act, M, K, ldx, off))
    buf = H.to_dev(padded(GU, ldx, off))[off:]
    Y, Xq = vq.silu_mul_quant(act, buf, buf[K:], M=M, K=K, ldx=ldx)
    Yh = H.host(Y)
    assert_close(Yh, oracle.silu_mul(G, U), TOL["silu"], "silu_mul Y")
    check_bytes(act, Xq, Yh)
    _, Xq2 = vq.silu_mul_quant(act, buf, buf[K:], M=M, K=K, ldx=ldx, want_y=False)
    for a, b in zip(planes(act, Xq, M, K), planes(act, Xq2, M, K)):
        assert np.array_equal(a, b), "bytes without Y"


def test_rmsnorm_special_rows():
    """A zero row (eps > 0: zero output, zero block), a constant row (exact
    closed form c / sqrt(c^2 + eps) with eps = 3, c = 1: 1/2), huge and tiny
    rows (no overflow in the sum of squares for |x| <= 1e17)."""
    K = 512
    X = np.zeros((4, K), np.float32)
    X[1] = 1.0
    X[2] = synth.normal(3400, (K,)) * np.float32(1e17)
    X[3] = synth.normal(3401, (K,)) * np.float32(1e-17)
    g = gamma_of(K, 3402)
    H.say("rmsnorm special rows")
    Y, Xq = vq.rmsnorm_quant(vq.Q8_K, H.to_dev(X), H.to_dev(g), 3.0)
    Yh = H.host(Y)
    assert not Yh[0].any()
    assert np.array_equal(Yh[1], g * np.float32(0.5))
    check_bytes(vq.Q8_K, Xq, Yh)
    Y2, _ = vq.rmsnorm_quant(vq.Q8_K, H.to_dev(X[2:]), H.to_dev(g), 0.0)
    assert_close(H.host(Y2), oracle.rmsnorm(X[2:], g, 0.0), tol_rmsnorm(K), "scaled rows")


def test_producer_errors():
    K = 512
    X = H.to_dev(np.ones((2, K), np.float32))
    g = H.to_dev(np.ones(K, np.float32))
    with pytest.raises(vq.VQError, match="INVALID_ARG"):
        vq.rmsnorm_quant(vq.Q8_K, X, g, -1.0)
    with pytest.raises(vq.VQError, match="UNSUPPORTED_TYPE"):
        vq.rmsnorm_quant(vq.Q4_K, X, g, 1e-6)
    with pytest.raises(vq.VQError, match="SHAPE"):
        vq.rmsnorm_quant(vq.Q8_K, X, g, 1e-6, M=2, K=300, ldx=K)
    with pytest.raises(vq.VQError, match="ALIAS"):
        vq.silu_mul_quant(vq.Q8_K, X, X, Y=X)


@pytest.mark.parametrize("which", ["Q4_K", "Q6_K"])
def test_decode_producer_into_gemv(which):
    """Decode: RMSNorm of the hidden row -> Q8_K -> Q4_K [9728, 2560], and
    SiLU-mul of gate/up rows -> Q8_K -> Q6_K [2560, 9728] (vq_gemm, M = 1):
    the products are bit-identical to the oracle GEMM on the oracle's bytes."""
    if which == "Q4_K":
        W = synth.tensor("decode_gemv", "Wa")
        N, K = W.shape
        x = synth.tensor("decode_gemv", "xa")[None, :]
        g = gamma_of(K, 3500)
        H.say("decode rmsnorm -> Q4_K gemv N=%d K=%d" % (N, K))
        Y, Xq = vq.rmsnorm_quant(vq.Q8_K, H.to_dev(x), H.to_dev(g), 1e-6)
        wtype = oracle.Q4_K
    else:
        W = synth.tensor("decode_gemv", "Wb")
        N, K = W.shape
        gu = synth.tensor("decode_gemv", "xb")
        u = synth.normal(3501, (K,))
        H.say("decode silu_mul -> Q6_K gemv N=%d K=%d" % (N, K))
        Y, Xq = vq.silu_mul_quant(vq.Q8_K, H.to_dev(gu[None, :]), H.to_dev(u[None, :]))
        wtype = oracle.Q6_K
    Yh = H.host(Y)
    act = check_bytes(vq.Q8_K, Xq, Yh)
    Wq = oracle.quantize_weights(wtype, W)
    y = vq.gemm(wtype, H.to_dev(Wq), N, K, vq.Q8_K, Xq, 1)
    H.assert_bitwise(H.host(y), oracle.gemm(wtype, Wq, N, K, act, nthreads=8), "producer -> " + which)
