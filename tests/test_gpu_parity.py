"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Every call goes through the C ABI (libvq.so via the thin binding).  Bar:
  * quantizer bytes, weight-encoder bytes, int32 sub-block sums (unit-scale
    probes) and routing: bit-exact;
  * GEMV, Q8_0 GEMM and grouped outputs: bit-identical to the oracle's
    fixed-order binary32 definition (stronger than the NMSE <= 1e-6 gate,
    which is checked too), and max relative error <= 5e-4 against the fp64
    dequantized product;
  * K-quant MFMA GEMM outputs (its own combine and accumulation order, and
    split K): NMSE <= 1e-6 against the oracle, max relative error <= 5e-4
    against fp64, two identical calls bitwise equal;
  * weighted expert sum: bit-identical to the oracle's sum of the GPU's Y.
Sizes span several tiles with ragged tails; full workload sizes are checked on
sampled outputs.
"""
import numpy as np
import pytest

import oracle
from oracle import ref_fp64
import synth
from tests import gpu_helpers as H
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import block_quantized_matmul_fp32_amd as vq  # noqa: E402

NMSE_MAX = 1e-6
REL_MAX = 5e-4

WTYPES = [oracle.Q4_K, oracle.Q6_K, oracle.Q8_0, oracle.Q5_K]
WNAME = {oracle.Q4_K: "Q4_K", oracle.Q6_K: "Q6_K", oracle.Q8_0: "Q8_0", oracle.Q5_K: "Q5_K"}


def oracle_act(wtype, X):
    return oracle.quantize_q8_1(X) if wtype == oracle.Q8_0 else oracle.quantize_q8k(X)


# ------------------------------------------------------------------ quantizers
def special_rows_q8k():
    rows = []
    r = np.full(256, 0.0, np.float32); r[0] = -127; r[1:7] = [0.5, 1.5, 2.5, -0.5, -1.5, 3.5]; rows.append(r)
    r = np.full(256, 1.0, np.float32); r[0] = 2.0; r[5] = -2.0; rows.append(r)
    rows.append(np.zeros(256, np.float32))
    rows.append(np.full(256, np.nan, np.float32))
    r = np.full(256, 0.25, np.float32); r[3] = np.array([0x3EE48B35], np.uint32).view(np.float32)[0]; rows.append(r)
    r = np.full(256, -3.0, np.float32); r[200] = 3.0; rows.append(r)  # ties at the end of the block
    return np.concatenate(rows)


def test_quantize_q8k_bitexact():
    M, K = 37, 2048
    X = synth.normal(1001, (M, K))
    X[0, :1536] = special_rows_q8k()
    X[1, 256:512] *= np.float32(1e-30)
    X[2, :256] = np.float32(7.0)
    for ldx, off in ((K, 0), (K + 4, 0), (K + 3, 1)):
        H.say("quantize_q8k M=%d K=%d ldx=%d offset=%d" % (M, K, ldx, off))
        Xp = np.zeros(M * ldx + off + 8, np.float32)
        view = np.lib.stride_tricks.as_strided(Xp[off:], (M, K), (4 * ldx, 4))
        view[:] = X
        Xd = H.to_dev(Xp)
        Xq = vq.quantize_act(vq.Q8_K, Xd[off:], M, K, ldx)
        qs, d, bs = H.planes_q8k(H.host(Xq), M, K)
        ref = oracle.quantize_q8k(X)
        assert np.array_equal(qs, ref.qs)
        assert np.array_equal(d.view(np.uint32), ref.d.view(np.uint32))
        assert np.array_equal(bs, ref.bsums)


def test_quantize_q8_1_bitexact():
    M, K = 29, 2080
    X = synth.normal(1002, (M, K))
    X[0, :32] = 0.0
    X[0, 32:64] = 0.0; X[0, 32] = 1.00048828125; X[0, 33] = X[0, 49] = 5.9604644775390625e-08
    X[1, :32] = 0.0; X[1, 0] = 127.0; X[1, 1:7] = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5]
    X[2, 64:96] = np.nan
    X[3] *= np.float32(2.0 ** -20)
    for ldx, off in ((K, 0), (K + 1, 3)):
        H.say("quantize_q8_1 M=%d K=%d ldx=%d offset=%d" % (M, K, ldx, off))
        Xp = np.zeros(M * ldx + off + 8, np.float32)
        view = np.lib.stride_tricks.as_strided(Xp[off:], (M, K), (4 * ldx, 4))
        view[:] = X
        Xq = vq.quantize_act(vq.Q8_1, H.to_dev(Xp)[off:], M, K, ldx)
        qs, d, s = H.planes_q8_1(H.host(Xq), M, K)
        ref = oracle.quantize_q8_1(X)
        assert np.array_equal(qs, ref.qs)
        assert np.array_equal(d, ref.d)
        assert np.array_equal(s, ref.s)
    assert s[0, 1] == 0x3C01  # butterfly-order case


@pytest.mark.parametrize("wtype", WTYPES)
def test_quantize_weights_bitexact(wtype):
    N, K = 67, 1024
    W = synth.normal(1003 + wtype, (N, K), 0.02)
    W[0] = 0.0
    W[1] = -0.01
    W[2] = 0.03
    W[3, :128] = 0.0
    W[4, ::3] = 0.0
    H.say("quantize_weights %s N=%d K=%d" % (WNAME[wtype], N, K))
    got = H.host(vq.quantize_weights(wtype, H.to_dev(W)))
    ref = oracle.quantize_weights(wtype, W).reshape(-1)
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------ GEMV
GEMV_SHAPES = {oracle.Q4_K: (300, 2560), oracle.Q6_K: (131, 1536), oracle.Q8_0: (300, 2080),
               oracle.Q5_K: (301, 4096)}


@pytest.mark.parametrize("wtype", WTYPES)
def test_gemv_bitexact_and_fused_bytes(wtype):
    N, K = GEMV_SHAPES[wtype]
    W = synth.normal(1100 + wtype, (N, K), 0.02)
    x = synth.normal(1110 + wtype, (K,))
    Wq = oracle.quantize_weights(wtype, W)
    act = oracle_act(wtype, x)
    y_ref = oracle.gemm(wtype, Wq, N, K, act)[0]
    H.say("gemv %s N=%d K=%d" % (WNAME[wtype], N, K))
    xq = H.to_dev(np.zeros(vq.act_bytes(vq.act_for(wtype), 1, K), np.uint8))
    y = H.to_dev(np.full(N, np.nan, np.float32))
    vq.gemv(wtype, H.to_dev(Wq), N, K, H.to_dev(x), y=y, xq_out=xq)
    H.assert_bitwise(H.host(y), y_ref, "gemv %s" % WNAME[wtype])
    assert np.array_equal(H.host(xq), H.pack_act(act, wtype)), "fused quantizer bytes"
    # the standalone quantizer writes the same bytes
    sq = vq.quantize_act(vq.act_for(wtype), H.to_dev(np.ascontiguousarray(x)),
                         Xq=H.to_dev(np.zeros(vq.act_bytes(vq.act_for(wtype), 1, K), np.uint8)))
    assert np.array_equal(H.host(sq), H.host(xq))
    r = ref_fp64.gemm_fp64(wtype, Wq, N, K, act)[0]
    assert ref_fp64.nmse(H.host(y), r) <= NMSE_MAX
    assert ref_fp64.max_rel_err(H.host(y), r)[0] <= REL_MAX


@pytest.mark.parametrize("wtype", WTYPES)
def test_gemv_edge_rows(wtype):
    """N = 1, a single block per row, and N around the rows-per-workgroup split."""
    qk = 32 if wtype == oracle.Q8_0 else 256
    for N, K in ((1, qk), (257, qk), (513, 4 * qk)):
        W = synth.normal((1200, N, K), (N, K), 0.02)
        x = synth.normal((1201, K), (K,))
        Wq = oracle.quantize_weights(wtype, W)
        y_ref = oracle.gemm(wtype, Wq, N, K, oracle_act(wtype, x))[0]
        H.say("gemv edge %s N=%d K=%d" % (WNAME[wtype], N, K))
        y = vq.gemv(wtype, H.to_dev(Wq), N, K, H.to_dev(x))
        H.assert_bitwise(H.host(y), y_ref, "gemv edge %s N=%d K=%d" % (WNAME[wtype], N, K))


@pytest.mark.parametrize("wtype", WTYPES)
def test_stream_probe_reads_only(wtype):
    """vq_stream_probe (the GEMV launch's streaming floor) runs on the decode
    shapes and a ragged one, and leaves its sink untouched."""
    import torch
    qk = 32 if wtype == oracle.Q8_0 else 256
    for N, K in ((2560, 9728 // qk * qk), (9728, 2560), (301, 17 * qk)):
        W = synth.normal((1190, wtype, N), (N, K), 0.02)
        Wq = H.to_dev(oracle.quantize_weights(wtype, W))
        sink = torch.full((N,), 7, dtype=torch.int32, device=H.dev())
        H.say("stream probe %s N=%d K=%d" % (WNAME[wtype], N, K))
        vq.stream_probe(wtype, Wq, N, K, sink)
        assert (H.host(sink) == 7).all()


def test_mfma_probe_runs():
    """vq_mfma_probe (the int8 MFMA ceiling) runs, leaves its sink untouched
    and reports 2*32*32*32 ops per MFMA: eight chains per wave, four waves
    per workgroup, two workgroups per CU."""
    import torch
    sink = torch.full((4,), 7, dtype=torch.int32, device=H.dev())
    H.say("mfma probe")
    ops = vq.mfma_probe(64, sink)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert ops == cus * 2 * 4 * 64 * 8 * 65536
    assert (H.host(sink) == 7).all()


def gemv_max_k(wtype):
    """Largest K the fused GEMV accepts (its weight row and quantized x must
    fit LDS), found from the library's host-side shape check, which rejects
    an oversized K before it looks at any pointer."""
    L = vq.lib()
    qk = 32 if wtype == oracle.Q8_0 else 256
    lo, hi = 1, 1 << 20  # blocks
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if L.vq_gemv(wtype, None, 1, mid * qk, None, None, None, None) == 4:  # VQ_ERR_SHAPE
            hi = mid - 1
        else:
            lo = mid
    return lo * qk


@pytest.mark.parametrize("wtype", WTYPES)
def test_gemv_max_k(wtype):
    """The GEMV at the largest accepted K (one row per workgroup, LDS nearly
    full), N = 1 and N = 300, and a three-row batch at that K (the GEMV
    kernel if its rows fit, else the MFMA GEMM): bit-identical to the oracle
    (the GEMV kernel, the Q8_0 GEMM) or within the GEMM tolerance; one block
    more is a shape error."""
    K = gemv_max_k(wtype)
    qk = 32 if wtype == oracle.Q8_0 else 256
    assert K >= 32768
    assert vq.lib().vq_gemv(wtype, None, 1, K + qk, None, None, None, None) == 4
    N = 300
    W = synth.normal((1250, wtype), (N, K), 0.02)
    X = synth.normal((1251, wtype), (3, K))
    Wq = oracle.quantize_weights(wtype, W)
    Wd = H.to_dev(Wq)
    act = oracle_act(wtype, X)
    Y_ref = oracle.gemm(wtype, Wq, N, K, act, nthreads=8)
    for n in (1, N):
        H.say("gemv max K %s N=%d K=%d" % (WNAME[wtype], n, K))
        y = vq.gemv(wtype, Wd[:n] if n == 1 else Wd, n, K, H.to_dev(X[0]))
        H.assert_bitwise(H.host(y), Y_ref[0, :n], "gemv max K %s N=%d" % (WNAME[wtype], n))
    H.say("gemm M=3 at max K %s K=%d" % (WNAME[wtype], K))
    at = vq.Q8_1 if wtype == oracle.Q8_0 else vq.Q8_K
    vq.reset_stats()
    Y = vq.gemm(wtype, Wd, N, K, at, H.to_dev(H.pack_act(act, wtype)), 3)
    if vq.get_stats()["gemm_skinny"]:
        H.assert_bitwise(H.host(Y), Y_ref, "gemm M=3 at max K %s" % WNAME[wtype])
    else:
        H.assert_gemm(wtype, H.host(Y), Y_ref, "gemm M=3 at max K %s" % WNAME[wtype],
                      ref_fp64.gemm_fp64(wtype, Wq, N, K, act))


# ------------------------------------------------------------------ GEMM
GEMM_SHAPES = {oracle.Q4_K: (150, 200, 1024), oracle.Q6_K: (150, 200, 1024), oracle.Q8_0: (150, 200, 2080),
               oracle.Q5_K: (150, 200, 1024)}


@pytest.mark.parametrize("wtype", WTYPES)
def test_gemm_parity(wtype):
    M, N, K = GEMM_SHAPES[wtype]
    W = synth.normal(1300 + wtype, (N, K), 0.02)
    X = synth.normal(1310 + wtype, (M, K))
    X[:, ::97] *= np.float32(20.0)
    Wq = oracle.quantize_weights(wtype, W)
    act = oracle_act(wtype, X)
    Y_ref = oracle.gemm(wtype, Wq, N, K, act, nthreads=8)
    H.say("gemm %s M=%d N=%d K=%d" % (WNAME[wtype], M, N, K))
    ldy = N + 7
    Yd = H.to_dev(np.full((M, ldy), np.nan, np.float32))
    vq.gemm(wtype, H.to_dev(Wq), N, K, vq.act_for(wtype), H.to_dev(H.pack_act(act, wtype)), M, Y=Yd, ldy=ldy)
    Yh = H.host(Yd)
    r = ref_fp64.gemm_fp64(wtype, Wq, N, K, act)
    H.assert_gemm(wtype, Yh[:, :N], Y_ref, "gemm %s" % WNAME[wtype], r)
    assert np.isnan(Yh[:, N:]).all(), "padding columns written"
    assert ref_fp64.nmse(Yh[:, :N], r) <= NMSE_MAX


# (weight type, M): N = 16400 is 129 column tiles of 128 (the last 16 wide);
# each M leaves a ragged last row tile of 128 (at M = 100 the only one).
LARGE_TILE_CASES = [(w, M) for w in (oracle.Q4_K, oracle.Q5_K) for M in (700, 1100, 300)] + \
                   [(oracle.Q6_K, M) for M in (700, 300, 100)]


@pytest.mark.parametrize("wtype,M", LARGE_TILE_CASES)
def test_gemm_large_tile_ragged(wtype, M):
    """Many column tiles with a ragged last row tile and column tile
    (N % 128 = 16); every output written, sampled outputs (whole first and
    last rows and columns) within the GEMM tolerance."""
    N, K = 16400, 512
    W = synth.normal(1350 + wtype, (N, K), 0.02)
    X = synth.normal(1360 + wtype + M, (M, K))
    Wq = oracle.quantize_weights(wtype, W)
    act = oracle_act(wtype, X)
    H.say("gemm large tile %s M=%d N=%d K=%d" % (WNAME[wtype], M, N, K))
    Yd = H.to_dev(np.full((M, N), np.nan, np.float32))
    vq.gemm(wtype, H.to_dev(Wq), N, K, vq.Q8_K, H.to_dev(H.pack_act(act, wtype)), M, Y=Yd)
    Yh = H.host(Yd)
    assert np.isfinite(Yh).all()
    rng = np.random.default_rng(1370)
    ms = np.concatenate([np.arange(M), rng.integers(0, M, 3000), np.full(N, M - 1)]).astype(np.int64)
    ns = np.concatenate([np.full(M, N - 1), rng.integers(0, N, 3000), np.arange(N)]).astype(np.int64)
    ref = oracle.gemm_sampled(wtype, Wq, N, K, act, ms, ns, nthreads=8)
    H.assert_gemm(wtype, Yh[ms, ns], ref, "gemm large tile %s" % WNAME[wtype],
                  H.fp64_cells(wtype, Wq, N, K, act, ms, ns))


@pytest.mark.parametrize("wtype,M,N,K", [(oracle.Q4_K, 700, 16400, 256), (oracle.Q5_K, 700, 16400, 256),
                                          (oracle.Q6_K, 700, 16400, 256), (oracle.Q8_0, 300, 200, 32),
                                          (oracle.Q8_0, 300, 200, 96)])
def test_gemm_single_step(wtype, M, N, K):
    """K of one super-block (one Q8_0 block, or three: a partial step): a
    single K step, nothing to split; sampled outputs (whole first and last
    rows and columns) bit-identical (Q8_0) or within the GEMM tolerance."""
    W = synth.normal((1460, wtype, K), (N, K), 0.02)
    X = synth.normal((1461, wtype, K), (M, K))
    Wq = oracle.quantize_weights(wtype, W)
    act = oracle_act(wtype, X)
    at = vq.Q8_1 if wtype == oracle.Q8_0 else vq.Q8_K
    H.say("gemm single step %s M=%d N=%d K=%d" % (WNAME[wtype], M, N, K))
    Yd = H.to_dev(np.full((M, N), np.nan, np.float32))
    vq.gemm(wtype, H.to_dev(Wq), N, K, at, H.to_dev(H.pack_act(act, wtype)), M, Y=Yd)
    Yh = H.host(Yd)
    assert np.isfinite(Yh).all()
    rng = np.random.default_rng(1462)
    ms = np.concatenate([np.arange(M), rng.integers(0, M, 2000), np.full(N, M - 1)]).astype(np.int64)
    ns = np.concatenate([np.full(M, N - 1), rng.integers(0, N, 2000), np.arange(N)]).astype(np.int64)
    ref = oracle.gemm_sampled(wtype, Wq, N, K, act, ms, ns, nthreads=8)
    H.assert_gemm(wtype, Yh[ms, ns], ref, "gemm single step %s K=%d" % (WNAME[wtype], K),
                  H.fp64_cells(wtype, Wq, N, K, act, ms, ns))


@pytest.mark.parametrize("wtype", WTYPES)
def test_gemm_row_blocks(wtype):
    """The MFMA GEMM split into launches of at most 200 or 256 activation rows
    (the path vq_gemm takes when one launch would address 2^31 activation
    bytes), with a ragged last block: Q8_0 gives the bytes of the single
    launch, the K-quants (whose K split depends on a block's rows) stay within
    the GEMM tolerance of it; sampled outputs against the oracle likewise."""
    M, N, K = 600, 16400, 512
    W = synth.normal(1380 + wtype, (N, K), 0.02)
    X = synth.normal(1390 + wtype, (M, K))
    Wq = oracle.quantize_weights(wtype, W)
    act = oracle_act(wtype, X)
    at = vq.Q8_1 if wtype == oracle.Q8_0 else vq.Q8_K
    Wd, Xd = H.to_dev(Wq), H.to_dev(H.pack_act(act, wtype))
    outs = []
    try:
        for rows in (0, 200, 256):
            H.say("gemm row blocks %s rows=%d M=%d N=%d K=%d" % (WNAME[wtype], rows, M, N, K))
            vq.set_gemm_row_block(rows)
            Yd = H.to_dev(np.full((M, N), np.nan, np.float32))
            vq.gemm(wtype, Wd, N, K, at, Xd, M, Y=Yd)
            outs.append(H.host(Yd))
    finally:
        vq.set_gemm_row_block(0)
    assert np.isfinite(outs[0]).all()
    for Y in outs[1:]:
        H.assert_gemm(wtype, Y, outs[0], "gemm row blocks %s" % WNAME[wtype])
    rng = np.random.default_rng(1395)
    ms = np.concatenate([np.arange(M), rng.integers(0, M, 2000)]).astype(np.int64)
    ns = np.concatenate([rng.integers(0, N, M), rng.integers(0, N, 2000)]).astype(np.int64)
    ref = oracle.gemm_sampled(wtype, Wq, N, K, act, ms, ns, nthreads=8)
    r64 = H.fp64_cells(wtype, Wq, N, K, act, ms, ns)
    for Y in outs:
        H.assert_gemm(wtype, Y[ms, ns], ref, "gemm row blocks %s vs oracle" % WNAME[wtype], r64)


@pytest.mark.parametrize("wtype", WTYPES)
def test_gemm_from_device_quantizer(wtype):
    """GPU quantize_act feeding GPU GEMM, decode-through-prefill M values."""
    N, K = 128, 512 if wtype != oracle.Q8_0 else 544
    W = synth.normal(1400 + wtype, (N, K), 0.02)
    Wq = oracle.quantize_weights(wtype, W)
    Wd = H.to_dev(Wq)
    for M in (1, 2, 7, 64, 129):
        X = synth.normal((1401, M), (M, K))
        H.say("gemm via device quantizer %s M=%d N=%d K=%d" % (WNAME[wtype], M, N, K))
        Xq = vq.quantize_act(vq.act_for(wtype), H.to_dev(X))
        Y = vq.gemm(wtype, Wd, N, K, vq.act_for(wtype), Xq, M)
        act = oracle_act(wtype, X)
        H.assert_gemm(wtype, H.host(Y), oracle.gemm(wtype, Wq, N, K, act), "M=%d" % M,
                      ref_fp64.gemm_fp64(wtype, Wq, N, K, act))


SKINNY_SHAPES = {oracle.Q4_K: (300, 2560), oracle.Q6_K: (131, 1536), oracle.Q8_0: (300, 2080),
                 oracle.Q5_K: (133, 2816)}


@pytest.mark.parametrize("wtype", WTYPES)
def test_gemm_small_batch(wtype):
    """M = 1..8 in one group and M > 8 in groups of four rows on the GEMV
    kernel reading the pre-quantized rows (the weights streamed once):
    bit-identical to the oracle and row m equal to the decode GEMV of x_m;
    the same M on the MFMA GEMM with the crossover set to 0: bit-identical
    (Q8_0) or within the GEMM tolerance; padding columns untouched."""
    N, K = SKINNY_SHAPES[wtype]
    W = synth.normal(1450 + wtype, (N, K), 0.02)
    Wq = oracle.quantize_weights(wtype, W)
    Wd = H.to_dev(Wq)
    ldy = N + 5
    try:
        for M in (1, 2, 3, 4, 5, 8, 9, 13, 16, 33):
            X = synth.normal((1451, wtype, M), (M, K))
            X[:, ::61] *= np.float32(15.0)
            act = oracle_act(wtype, X)
            ref = oracle.gemm(wtype, Wq, N, K, act, nthreads=8)
            r64 = ref_fp64.gemm_fp64(wtype, Wq, N, K, act)
            Xq = H.to_dev(H.pack_act(act, wtype))
            Yskinny = None
            for max_m, skinny in ((64, 1), (0, 0)):
                H.say("gemm small batch %s M=%d N=%d K=%d crossover %d" % (WNAME[wtype], M, N, K, max_m))
                vq.set_small_batch_max(wtype, max_m)
                vq.reset_stats()
                Yd = H.to_dev(np.full((M, ldy), np.nan, np.float32))
                vq.gemm(wtype, Wd, N, K, vq.act_for(wtype), Xq, M, Y=Yd, ldy=ldy)
                Yh = H.host(Yd)
                assert vq.get_stats()["gemm_skinny"] == skinny
                if skinny:
                    H.assert_bitwise(Yh[:, :N], ref, "M=%d crossover %d" % (M, max_m))
                    Yskinny = Yh
                else:
                    H.assert_gemm(wtype, Yh[:, :N], ref, "M=%d crossover %d" % (M, max_m), r64)
                assert np.isnan(Yh[:, N:]).all(), "padding columns written"
            for m in sorted({0, M - 1}):
                y = vq.gemv(wtype, Wd, N, K, H.to_dev(np.ascontiguousarray(X[m])))
                H.assert_bitwise(H.host(y), Yskinny[m, :N], "gemv row %d vs gemm M=%d" % (m, M))
    finally:
        vq.set_small_batch_max(wtype, -1)


@pytest.mark.parametrize("wtype", WTYPES)
def test_random_byte_blocks(wtype):
    """Random block bytes (random scales, mins, quants incl. negative Q6_K scales),
    binary16 d in [2^-10, 1]."""
    rng = np.random.default_rng(1500 + wtype)
    N, K, M = 96, 1024, 40
    bb = oracle.BLOCK_BYTES[wtype]
    nb = K // oracle.BLOCK_ELEMS[wtype]
    Wq = rng.integers(0, 256, (N, nb, bb), dtype=np.uint8)
    dv = (2.0 ** rng.uniform(-10, 0, (N, nb, 2))).astype(np.float16).view(np.uint8).reshape(N, nb, 4)
    if wtype in (oracle.Q4_K, oracle.Q5_K):
        Wq[..., 0:4] = dv
    elif wtype == oracle.Q6_K:
        Wq[..., 208:210] = dv[..., 0:2]
    else:
        Wq[..., 0:2] = dv[..., 0:2]
    Wq = Wq.reshape(N, -1)
    X = synth.normal(1501 + wtype, (M, K))
    act = oracle_act(wtype, X)
    H.say("random bytes %s M=%d N=%d K=%d" % (WNAME[wtype], M, N, K))
    Y = vq.gemm(wtype, H.to_dev(Wq), N, K, vq.act_for(wtype), H.to_dev(H.pack_act(act, wtype)), M)
    H.assert_gemm(wtype, H.host(Y), oracle.gemm(wtype, Wq, N, K, act), "gemm random bytes",
                  ref_fp64.gemm_fp64(wtype, Wq, N, K, act))
    y = vq.gemv(wtype, H.to_dev(Wq), N, K, H.to_dev(X[0]))
    H.assert_bitwise(H.host(y), oracle.gemm(wtype, Wq, N, K, oracle_act(wtype, X[:1]))[0], "gemv random bytes")


def test_unit_scale_probes_exact_int32():
    """d = 1, one sub-block scale 1, activations with iscale = 1: outputs are the
    exact int32 sub-block sums (GEMV and GEMM)."""
    a = ((np.arange(256) * 37) % 255 - 127).astype(np.float32)
    rng = np.random.default_rng(1600)
    q = rng.integers(0, 16, 256)
    blocks = []
    for j in range(8):
        sc = np.zeros(8, np.int32); sc[j] = 1
        blocks.append(oracle.q4k_build(0x3C00, 0, sc, np.zeros(8, np.int32), q))
    Wq = np.stack(blocks)
    want = np.array([sum(int(q[i]) * int(a[i]) for i in range(32 * j, 32 * j + 32)) for j in range(8)],
                    np.float32)
    H.say("unit-scale probes Q4_K")
    y = vq.gemv(vq.Q4_K, H.to_dev(Wq), 8, 256, H.to_dev(a))
    assert np.array_equal(H.host(y), want)
    Xq = vq.quantize_act(vq.Q8_K, H.to_dev(np.stack([a] * 3)))
    Y = vq.gemm(vq.Q4_K, H.to_dev(Wq), 8, 256, vq.Q8_K, Xq, 3)
    assert np.array_equal(H.host(Y), np.stack([want] * 3))
    q6 = rng.integers(0, 64, 256)
    blocks = []
    for j in range(16):
        sc = np.zeros(16, np.int32); sc[j] = 1
        blocks.append(oracle.q6k_build(0x3C00, sc, q6))
    Wq = np.stack(blocks)
    want = np.array([sum((int(q6[i]) - 32) * int(a[i]) for i in range(16 * j, 16 * j + 16)) for j in range(16)],
                    np.float32)
    H.say("unit-scale probes Q6_K")
    y = vq.gemv(vq.Q6_K, H.to_dev(Wq), 16, 256, H.to_dev(a))
    assert np.array_equal(H.host(y), want)
    Y = vq.gemm(vq.Q6_K, H.to_dev(Wq), 16, 256, vq.Q8_K, Xq, 3)
    assert np.array_equal(H.host(Y), np.stack([want] * 3))
    # Q5_K: quants 0..31 (fifth bits set), GEMV, GEMV-kernel batch and MFMA GEMM (70 rows)
    q5 = rng.integers(0, 32, 256)
    blocks = []
    for j in range(8):
        sc = np.zeros(8, np.int32); sc[j] = 1
        blocks.append(oracle.q5k_build(0x3C00, 0, sc, np.zeros(8, np.int32), q5))
    for j in range(8):  # scale 63 = 3 * 16 + 3 * 4 + 3: every base-4 digit plane at its largest
        sc = np.zeros(8, np.int32); sc[j] = 63
        blocks.append(oracle.q5k_build(0x3C00, 0, sc, np.zeros(8, np.int32), q5))
    Wq = np.stack(blocks)
    I = np.array([sum(int(q5[i]) * int(a[i]) for i in range(32 * j, 32 * j + 32)) for j in range(8)], np.int64)
    want = np.concatenate([I, 63 * I]).astype(np.float32)
    assert np.array_equal(want.astype(np.int64), np.concatenate([I, 63 * I]))  # exact in binary32
    H.say("unit-scale probes Q5_K")
    y = vq.gemv(vq.Q5_K, H.to_dev(Wq), 16, 256, H.to_dev(a))
    assert np.array_equal(H.host(y), want)
    Y = vq.gemm(vq.Q5_K, H.to_dev(Wq), 16, 256, vq.Q8_K, Xq, 3)
    assert np.array_equal(H.host(Y), np.stack([want] * 3))
    Xq70 = vq.quantize_act(vq.Q8_K, H.to_dev(np.stack([a] * 70)))
    Y = vq.gemm(vq.Q5_K, H.to_dev(Wq), 16, 256, vq.Q8_K, Xq70, 70)
    assert np.array_equal(H.host(Y), np.stack([want] * 70))
    # Q8_0: d = 1 weights, activations with amax 127 give d = 1
    a32 = ((np.arange(64) * 29) % 255 - 127).astype(np.float32)
    a32[0] = 127.0; a32[32] = -127.0
    qw = rng.integers(-127, 128, (4, 64)).astype(np.int8)
    Wq = np.zeros((4, 2, 34), np.uint8)
    Wq[:, :, 0:2] = np.array([0x3C00], np.uint16).view(np.uint8)
    Wq[:, :, 2:] = qw.reshape(4, 2, 32).view(np.uint8)
    want = (qw.astype(np.int64) @ a32.astype(np.int64)).astype(np.float32)
    H.say("unit-scale probes Q8_0")
    y = vq.gemv(vq.Q8_0, H.to_dev(Wq.reshape(4, -1)), 4, 64, H.to_dev(a32))
    assert np.array_equal(H.host(y), want)


def unit_probe_blocks(wtype, rng):
    """Blocks with d = 1, dmin = 0 and one sub-block scale 1 (the rest 0), one
    block per sub-block, and the quants; the output of row j is then the exact
    int32 sum over sub-block j of q (Q6_K: q - 32) times the activation bytes."""
    if wtype == oracle.Q6_K:
        q = rng.integers(0, 64, 256)
        blocks = []
        for j in range(16):
            sc = np.zeros(16, np.int32); sc[j] = 1
            blocks.append(oracle.q6k_build(0x3C00, sc, q))
        return np.stack(blocks), q - 32, 16
    hi = 32 if wtype == oracle.Q5_K else 16
    q = rng.integers(0, hi, 256)
    build = oracle.q5k_build if wtype == oracle.Q5_K else oracle.q4k_build
    blocks = []
    for j in range(8):
        sc = np.zeros(8, np.int32); sc[j] = 1
        blocks.append(build(0x3C00, 0, sc, np.zeros(8, np.int32), q))
    return np.stack(blocks), q, 32


@pytest.mark.parametrize("wtype", [oracle.Q4_K, oracle.Q6_K, oracle.Q5_K])
def test_unit_scale_probes_mfma_split_k(wtype):
    """The int32 sub-block sums through the MFMA GEMM (crossover 0), over one
    super-block and over 16 super-blocks with K split across workgroups (one
    output tile, so the plan splits K): every output the exact integer.  With
    d = da = 1 and dmin = 0 each step adds an integer below 2^24, so every
    binary32 operation of the combine, the accumulation and the split-K sum
    is exact."""
    rng = np.random.default_rng(1650 + wtype)
    blocks, qv, sub = unit_probe_blocks(wtype, rng)
    N = blocks.shape[0]
    a = ((np.arange(256) * 37) % 255 - 127).astype(np.float32)
    I = np.array([int(np.dot(qv[sub * j: sub * j + sub].astype(np.int64), a[sub * j: sub * j + sub].astype(np.int64)))
                  for j in range(N)], np.int64)
    try:
        vq.set_small_batch_max(wtype, 0)
        for nsb, M in ((1, 3), (1, 70), (16, 70), (16, 129)):
            K = 256 * nsb
            Wq = np.concatenate([blocks] * nsb, axis=1)  # row j: nsb copies of its probe block
            X = np.tile(a, (M, nsb))
            want = (nsb * I).astype(np.float32)
            assert np.array_equal(want.astype(np.int64), nsb * I)
            H.say("unit-scale probes MFMA %s M=%d K=%d" % (WNAME[wtype], M, K))
            Xq = vq.quantize_act(vq.Q8_K, H.to_dev(X))
            if nsb > 1:
                assert vq.gemm_workspace(wtype, M, N, K) > 0, "the plan splits K here"
            Y = vq.gemm(wtype, H.to_dev(Wq), N, K, vq.Q8_K, Xq, M)
            assert np.array_equal(H.host(Y), np.stack([want] * M)), "M=%d K=%d" % (M, K)
    finally:
        vq.set_small_batch_max(wtype, -1)


@pytest.mark.parametrize("wtype", [oracle.Q4_K, oracle.Q6_K, oracle.Q5_K])
def test_gemm_split_k_workspace(wtype):
    """Split K on a grid of 10 output tiles with 16 K steps: the planned
    workspace, a workspace holding only two splits, and none (no split) all
    give outputs within the GEMM tolerance of the oracle; two calls with the
    same workspace size are bitwise equal; the arrival counters are zero
    after every call."""
    M, N, K = 256, 640, 4096
    W = synth.normal(1670 + wtype, (N, K), 0.02)
    X = synth.normal(1671 + wtype, (M, K))
    X[:, ::97] *= np.float32(20.0)
    Wq = oracle.quantize_weights(wtype, W)
    act = oracle_act(wtype, X)
    ref = oracle.gemm(wtype, Wq, N, K, act, nthreads=8)
    r64 = ref_fp64.gemm_fp64(wtype, Wq, N, K, act)
    Wd, Xq = H.to_dev(Wq), H.to_dev(H.pack_act(act, wtype))
    need = vq.gemm_workspace(wtype, M, N, K)
    tiles = ((N + 127) // 128) * ((M + 127) // 128)
    cnt_bytes = 65536  # the arrival counters' fixed region
    part_tile = 128 * 128 * 4  # one binary32 partial tile of 128 x 128 outputs
    assert need > cnt_bytes + tiles * 2 * part_tile, "the plan takes more than two splits"
    two = cnt_bytes + tiles * 2 * part_tile
    import torch
    outs = {}
    for name, nbytes in (("planned", need), ("two splits", two), ("none", 0)):
        ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=H.dev()) if nbytes else None
        runs = []
        for rep in range(2):
            H.say("gemm split K %s workspace %s (%d bytes) run %d" % (WNAME[wtype], name, nbytes, rep))
            Yd = H.to_dev(np.full((M, N), np.nan, np.float32))
            vq.gemm(wtype, Wd, N, K, vq.Q8_K, Xq, M, Y=Yd, ws=ws)
            runs.append(H.host(Yd))
            if ws is not None:
                assert not H.host(ws[:cnt_bytes]).any(), "arrival counters left non-zero"
        assert np.array_equal(H.bits(runs[0]), H.bits(runs[1])), "two identical calls differ (%s)" % name
        H.assert_close(runs[0], ref, "split K %s %s" % (WNAME[wtype], name), r64)
        outs[name] = runs[0]
    H.assert_close(outs["planned"], outs["none"], "split vs no split %s" % WNAME[wtype])


@pytest.mark.parametrize("wtype", [oracle.Q4_K, oracle.Q6_K])
def test_gemm_workspace_reused_across_shapes(wtype):
    """One workspace for a 10-tile call split eight ways, then an 80-tile call
    split three ways: the second call's counters (80 of them) must not meet
    the first call's partial tiles, so both outputs meet the tolerance."""
    import torch
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=H.dev())
    for (M, N, K), seed in (((256, 640, 4096), 1680), ((512, 2560, 2048), 1690)):
        assert vq.gemm_workspace(wtype, M, N, K) > 0
        W = synth.normal((seed, wtype), (N, K), 0.02)
        X = synth.normal((seed + 1, wtype), (M, K))
        Wq = oracle.quantize_weights(wtype, W)
        act = oracle_act(wtype, X)
        H.say("gemm reused workspace %s M=%d N=%d K=%d" % (WNAME[wtype], M, N, K))
        Y = vq.gemm(wtype, H.to_dev(Wq), N, K, vq.Q8_K, H.to_dev(H.pack_act(act, wtype)), M, ws=ws)
        H.assert_close(H.host(Y), oracle.gemm(wtype, Wq, N, K, act, nthreads=8),
                       "reused workspace %s M=%d" % (WNAME[wtype], M), ref_fp64.gemm_fp64(wtype, Wq, N, K, act))


@pytest.mark.parametrize("wtype,M,N,K,parts", [(oracle.Q4_K, 200, 9728, 2560, 3), (oracle.Q5_K, 300, 8192, 2560, 2)])
def test_gemm_split_two_per_cu(wtype, M, N, K, parts):
    """Grids of at most one tile per CU that the plan splits into two
    workgroups per CU (152 tiles in three parts, 192 tiles in two), with a
    ragged last row tile: every output written, sampled outputs (whole first
    and last rows and columns) within the GEMM tolerance, two calls bitwise
    equal."""
    tiles = ((N + 127) // 128) * ((M + 127) // 128)
    assert vq.gemm_workspace(wtype, M, N, K) == 65536 + tiles * parts * 128 * 128 * 4
    W = synth.normal((1710, wtype), (N, K), 0.02)
    X = synth.normal((1711, wtype, M), (M, K))
    Wq = oracle.quantize_weights(wtype, W)
    del W
    act = oracle_act(wtype, X)
    Wd, Xq = H.to_dev(Wq), H.to_dev(H.pack_act(act, wtype))
    runs = []
    for rep in range(2):
        H.say("gemm two per CU %s M=%d N=%d K=%d run %d" % (WNAME[wtype], M, N, K, rep))
        Yd = H.to_dev(np.full((M, N), np.nan, np.float32))
        vq.gemm(wtype, Wd, N, K, vq.Q8_K, Xq, M, Y=Yd)
        runs.append(H.host(Yd))
    Yh = runs[0]
    assert np.isfinite(Yh).all(), "every output written"
    assert np.array_equal(H.bits(runs[1]), H.bits(Yh)), "two identical calls differ"
    rng = np.random.default_rng(1712)
    ms = np.concatenate([np.arange(M), rng.integers(0, M, 3000), np.full(N, M - 1)]).astype(np.int64)
    ns = np.concatenate([np.full(M, N - 1), rng.integers(0, N, 3000), np.arange(N)]).astype(np.int64)
    ref = oracle.gemm_sampled(wtype, Wq, N, K, act, ms, ns, nthreads=8)
    H.assert_gemm(wtype, Yh[ms, ns], ref, "gemm two per CU %s" % WNAME[wtype],
                  H.fp64_cells(wtype, Wq, N, K, act, ms, ns))


def test_determinism_and_witness():
    N, K, M = 256, 2560, 130
    W = synth.normal(1700, (N, K), 0.02)
    Wq = H.to_dev(oracle.quantize_weights(oracle.Q4_K, W))
    X = H.to_dev(synth.normal(1701, (M, K)))
    vq.reset_stats()
    H.say("determinism Q4_K")
    Xq = vq.quantize_act(vq.Q8_K, X)
    Y1 = H.host(vq.gemm(vq.Q4_K, Wq, N, K, vq.Q8_K, Xq, M))
    Y2 = H.host(vq.gemm(vq.Q4_K, Wq, N, K, vq.Q8_K, Xq, M))
    y1 = H.host(vq.gemv(vq.Q4_K, Wq, N, K, X[0]))
    y2 = H.host(vq.gemv(vq.Q4_K, Wq, N, K, X[0]))
    assert np.array_equal(Y1.view(np.uint32), Y2.view(np.uint32))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    st = vq.get_stats()
    assert st["quantize_q8k"] == 1 and st["gemm_q4k"] == 2 and st["gemv_q4k"] == 2
    assert st["gemm_q6k"] == 0 and st["gemv_q8_0"] == 0
    # decode through prefill: the GEMM row 0 is the GEMV within the GEMM
    # tolerance; the GEMV-kernel arm of vq_gemm gives the GEMV's bits
    H.assert_close(Y1[0], y1, "gemv vs gemm row 0")
    Xq4 = vq.quantize_act(vq.Q8_K, X[:4].contiguous())  # the planar layout depends on M
    Ys = H.host(vq.gemm(vq.Q4_K, Wq, N, K, vq.Q8_K, Xq4, 4))
    H.assert_bitwise(y1, Ys[0], "gemv vs small-batch row 0")


# ------------------------------------------------------------------ grouped
def grouped_fp64(wtype, Wq, E, N, K, act, ids, per_row=False):
    """fp64 dequantized products of every (token, slot) pair: [T, top_k, N]."""
    T, top_k = ids.shape
    A = ref_fp64.dequant_act(act)
    Wd = ref_fp64.dequant_weights(wtype, Wq, E * N, K).reshape(E, N, K)
    out = np.zeros((T, top_k, N))
    for t in range(T):
        for s_ in range(top_k):
            e = int(ids[t, s_])
            if 0 <= e < E:
                out[t, s_] = Wd[e] @ A[t * top_k + s_ if per_row else t]
    return out


def run_grouped(E, N, K, T, top_k, ids, seed, wtype=oracle.Q4_K, per_row=False):
    W = np.stack([synth.normal((seed, e), (N, K), 0.02) for e in range(E)])
    Wq = np.stack([oracle.quantize_weights(wtype, W[e]) for e in range(E)]).reshape(E * N, -1)
    X = synth.normal(seed + 1, (T * top_k if per_row else T, K))
    logits = synth.normal(seed + 2, (T, top_k))
    z = np.exp(logits - logits.max(1, keepdims=True))
    rw = (z / z.sum(1, keepdims=True)).astype(np.float32)
    act = oracle_act(wtype, X)
    at = vq.Q8_1 if wtype == oracle.Q8_0 else vq.Q8_K
    H.say("grouped %s per_row=%d E=%d N=%d K=%d T=%d top_k=%d" % (WNAME[wtype], per_row, E, N, K, T, top_k))
    Xq = vq.quantize_act(at, H.to_dev(X))
    Yd = H.to_dev(np.full((T, top_k, N), np.nan, np.float32))
    Sd = H.to_dev(np.full((T, N), np.nan, np.float32))
    Y, Ysum, ws = vq.gemm_grouped(wtype, H.to_dev(Wq), E, N, K, at, Xq, T, H.to_dev(ids), top_k,
                                  route_w=H.to_dev(rw), Y=Yd, Ysum=Sd, per_row=per_row)
    return Wq, act, rw, Y, Ysum, ws


@pytest.mark.parametrize("case", ["uniform", "skewed"])
def test_grouped_small(case):
    E, N, K, top_k = 16, 80, 512, 4
    if case == "uniform":
        T = 50
        ids = synth.random_ids(1800, T, E, top_k)
    else:
        # expert 0 empty, expert 1 in every token (rows over several tiles),
        # expert 2 once
        T = 150
        hint = np.ones(E); hint[0] = 0; hint[1] = 1e6; hint[2] = 0
        ids = synth.skewed_ids(1801, T, E, top_k, hint)
        ids[5, 3] = 2 if 2 not in ids[5] else ids[5, 3]
    Wq, act, rw, Y, Ysum, ws = run_grouped(E, N, K, T, top_k, ids, 1810)
    counts, offsets, lst = vq.grouped_ws_views(ws, E, T, top_k)
    c_ref, o_ref, l_ref = oracle.route(ids, E)
    assert np.array_equal(H.host(counts), c_ref)
    assert np.array_equal(H.host(offsets), o_ref)
    assert np.array_equal(H.host(lst), l_ref)
    Y_ref = oracle.gemm_grouped(oracle.Q4_K, Wq, E, N, K, act, ids, nthreads=8)
    Yh = H.host(Y)
    H.assert_gemm(oracle.Q4_K, Yh, Y_ref, "grouped Y", grouped_fp64(oracle.Q4_K, Wq, E, N, K, act, ids))
    H.assert_bitwise(H.host(Ysum), oracle.weighted_sum(Yh, rw), "weighted sum of the GPU's Y")
    # each slot equals a dense GEMM of its expert
    e = int(ids[0, 0])
    dense = oracle.gemm(oracle.Q4_K, Wq[e * N:(e + 1) * N], N, K, act)
    H.assert_close(Yh[0, 0], dense[0], "slot vs dense")
    if case == "skewed":
        assert int(H.host(counts)[1]) == T and int(H.host(counts)[0]) == 0
    # swapped ids must change the output
    ids2 = ids.copy(); ids2[:, [0, 1]] = ids2[:, [1, 0]]
    _, _, _, Y2, _, _ = run_grouped(E, N, K, T, top_k, ids2, 1810)
    assert not np.array_equal(H.host(Y2), Yh)


@pytest.mark.parametrize("per_row", [False, True])
@pytest.mark.parametrize("wtype", WTYPES)
def test_grouped_types_and_arms(wtype, per_row):
    """Every weight type in both arms (broadcast: x_t; per-row: x_(t*top_k+s)):
    routing and the weighted sum bit-identical to the oracle, Y bit-identical
    (Q8_0) or within the GEMM tolerance."""
    E, N, K, top_k, T = 10, 48, 512, 3, 70
    ids = synth.random_ids(1850 + wtype, T, E, top_k)
    vq.reset_stats()
    Wq, act, rw, Y, Ysum, ws = run_grouped(E, N, K, T, top_k, ids, 1860, wtype, per_row)
    counts, offsets, lst = vq.grouped_ws_views(ws, E, T, top_k)
    c_ref, o_ref, l_ref = oracle.route(ids, E)
    assert np.array_equal(H.host(counts), c_ref) and np.array_equal(H.host(lst), l_ref)
    Y_ref = oracle.gemm_grouped(wtype, Wq, E, N, K, act, ids, nthreads=8, per_row=per_row)
    Yh = H.host(Y)
    H.assert_gemm(wtype, Yh, Y_ref, "grouped %s per_row=%d" % (WNAME[wtype], per_row),
                  grouped_fp64(wtype, Wq, E, N, K, act, ids, per_row))
    H.assert_bitwise(H.host(Ysum), oracle.weighted_sum(Yh, rw), "weighted sum of the GPU's Y")
    st = vq.get_stats()
    key = {oracle.Q4_K: "gemm_grouped_q4k", oracle.Q6_K: "gemm_grouped_q6k", oracle.Q8_0: "gemm_grouped_q8_0",
           oracle.Q5_K: "gemm_grouped_q5k"}[wtype]
    assert st[key] == 1 and st["gemm_grouped_rows"] == int(per_row) and st["route"] == 1


def test_grouped_route_unstaged_scan():
    """Many experts (1000 tokens x top-4 over 1024 experts, routed by the
    single-workgroup kernel with its per-wave counts for every expert):
    routing bit-identical to the oracle, Y within the GEMM tolerance."""
    E, N, K, T, top_k = 1024, 16, 256, 1000, 4
    ids = synth.random_ids(1880, T, E, top_k)
    Wq, act, rw, Y, Ysum, ws = run_grouped(E, N, K, T, top_k, ids, 1890)
    counts, offsets, lst = vq.grouped_ws_views(ws, E, T, top_k)
    c_ref, o_ref, l_ref = oracle.route(ids, E)
    assert np.array_equal(H.host(counts), c_ref)
    assert np.array_equal(H.host(offsets), o_ref)
    assert np.array_equal(H.host(lst), l_ref)
    Y_ref = oracle.gemm_grouped(oracle.Q4_K, Wq, E, N, K, act, ids, nthreads=8)
    Yh = H.host(Y)
    H.assert_gemm(oracle.Q4_K, Yh, Y_ref, "grouped Y (unstaged routing scan)")
    H.assert_bitwise(H.host(Ysum), oracle.weighted_sum(Yh, rw), "weighted sum of the GPU's Y")


@pytest.mark.parametrize("E,T,top_k,skew", [(16, 1100, 8, False), (1024, 1100, 8, False),
                                             (8, 1024, 8, True), (9, 1025, 8, True),
                                             (16, 4200, 2, False), (1024, 4200, 2, False),
                                             (64, 600, 16, False), (1024, 700, 16, True)])
def test_grouped_route_size_paths(E, T, top_k, skew):
    """Routing on every path: 1100 x top-8 (18 chunks of 64 tokens) takes the
    two-launch path (count, then one workgroup per chunk scanning and
    placing) with 16 or 1024 experts; 1024 x 8 pairs almost all on one
    expert (repeated ids) fill the single-workgroup kernel to its limit of
    8192 pairs, and one token more goes to the two-launch path; 4200 x top-2
    (66 chunks) takes the three-launch path with its chunk table staged in
    LDS (16 experts) or read in global memory (1024 experts); 600 and 700
    tokens x top-16 fill each chunk of the count kernel (1024 pairs, four
    rounds per wave), the second almost all on one expert.  Counts,
    offsets and the list bit-identical to the oracle, Y within the GEMM
    tolerance."""
    N, K = 16, 256
    if skew:
        ids = np.zeros((T, top_k), np.int32)
        ids[::37, 1] = 1
        ids[5::41, 2] = E - 1
    else:
        ids = synth.random_ids(1940 + E, T, E, top_k)
    Wq, act, rw, Y, Ysum, ws = run_grouped(E, N, K, T, top_k, ids, 1950)
    counts, offsets, lst = vq.grouped_ws_views(ws, E, T, top_k)
    c_ref, o_ref, l_ref = oracle.route(ids, E)
    assert np.array_equal(H.host(counts), c_ref)
    assert np.array_equal(H.host(offsets), o_ref)
    assert np.array_equal(H.host(lst), l_ref)
    Y_ref = oracle.gemm_grouped(oracle.Q4_K, Wq, E, N, K, act, ids, nthreads=8)
    Yh = H.host(Y)
    H.assert_gemm(oracle.Q4_K, Yh, Y_ref, "grouped Y (routing size paths)")
    H.assert_bitwise(H.host(Ysum), oracle.weighted_sum(Yh, rw), "weighted sum of the GPU's Y")


@pytest.mark.parametrize("per_row", [False, True])
def test_grouped_tile_launches(per_row):
    """The Q8_0 grouped GEMM split into launches of one or two routed tiles
    (the row-block hook; large calls launch once per 32768 tiles) gives the
    bytes of the single launch, and they match the oracle."""
    E, N, K, T, top_k = 12, 64, 512, 150, 4
    ids = synth.random_ids(1870, T, E, top_k)
    outs = []
    try:
        for rows in (0, 96, 200):
            vq.set_gemm_row_block(rows)
            Wq, act, rw, Y, Ysum, ws = run_grouped(E, N, K, T, top_k, ids, 1875, wtype=oracle.Q8_0,
                                                   per_row=per_row)
            outs.append((H.host(Y), H.host(Ysum)))
    finally:
        vq.set_gemm_row_block(0)
    for Yb, Sb in outs[1:]:
        H.assert_bitwise(Yb, outs[0][0], "grouped tile launches Y")
        H.assert_bitwise(Sb, outs[0][1], "grouped tile launches Ysum")
    Y_ref = oracle.gemm_grouped(oracle.Q8_0, Wq, E, N, K, act, ids, nthreads=8, per_row=per_row)
    H.assert_bitwise(outs[1][0], Y_ref, "grouped tile launches vs oracle")


# rows per expert r -> routed tile height 32 (r = 4, 16), 64 (32), 96 (64; 128 in two tiles)
@pytest.mark.parametrize("wtype", [oracle.Q4_K, oracle.Q6_K, oracle.Q5_K])
@pytest.mark.parametrize("rows", [4, 16, 32, 64, 128])
def test_grouped_rows_per_expert(wtype, rows):
    """Uniform top-4 routing over 32 experts at 4, 16, 32, 64 and 128 rows per
    expert (every routed tile height, ragged last tiles): routing and the
    weighted sum bit-identical, Y within the GEMM tolerance of the oracle and
    the fp64 product."""
    E, N, K, top_k = 32, 256, 512, 4
    T = rows * E // top_k
    ids = synth.random_ids((1940, rows), T, E, top_k)
    Wq, act, rw, Y, Ysum, ws = run_grouped(E, N, K, T, top_k, ids, 1945 + rows, wtype)
    counts, offsets, lst = vq.grouped_ws_views(ws, E, T, top_k)
    c_ref, o_ref, l_ref = oracle.route(ids, E)
    assert np.array_equal(H.host(counts), c_ref) and np.array_equal(H.host(offsets), o_ref)
    assert np.array_equal(H.host(lst), l_ref)
    Y_ref = oracle.gemm_grouped(wtype, Wq, E, N, K, act, ids, nthreads=8)
    Yh = H.host(Y)
    H.assert_close(Yh, Y_ref, "grouped %s %d rows per expert" % (WNAME[wtype], rows),
                   grouped_fp64(wtype, Wq, E, N, K, act, ids))
    H.assert_bitwise(H.host(Ysum), oracle.weighted_sum(Yh, rw), "weighted sum of the GPU's Y")


@pytest.mark.parametrize("E,top_k", [(1, 1), (4, 4)])
def test_grouped_degenerate_routing(E, top_k):
    """One expert at top-1 (the grouped call is the dense GEMM of that expert,
    over several routed tiles; the dense call agrees to the GEMM tolerance)
    and top_k = E (every token in every expert): routing and the weighted sum
    bit-identical to the oracle, Y within the GEMM tolerance."""
    N, K, T = 64, 512, 300
    ids = np.tile(np.arange(top_k, dtype=np.int32), (T, 1))
    if E > 1:
        ids = synth.random_ids(1920, T, E, top_k)  # a permutation of all E per token
    Wq, act, rw, Y, Ysum, ws = run_grouped(E, N, K, T, top_k, ids, 1925)
    counts, offsets, lst = vq.grouped_ws_views(ws, E, T, top_k)
    c_ref, o_ref, l_ref = oracle.route(ids, E)
    assert np.array_equal(H.host(counts), c_ref) and np.array_equal(H.host(lst), l_ref)
    assert (H.host(counts) == T).all()
    Y_ref = oracle.gemm_grouped(oracle.Q4_K, Wq, E, N, K, act, ids, nthreads=8)
    Yh = H.host(Y)
    H.assert_gemm(oracle.Q4_K, Yh, Y_ref, "grouped degenerate E=%d top_k=%d" % (E, top_k),
                  grouped_fp64(oracle.Q4_K, Wq, E, N, K, act, ids))
    H.assert_bitwise(H.host(Ysum), oracle.weighted_sum(Yh, rw), "weighted sum of the GPU's Y")
    if E == 1:
        dense = vq.gemm(vq.Q4_K, H.to_dev(Wq), N, K, vq.Q8_K, H.to_dev(H.pack_act(act, oracle.Q4_K)), T)
        H.assert_close(H.host(dense), Yh[:, 0, :], "dense GEMM vs grouped E=1")


def test_grouped_out_of_range_ids_skipped():
    """A pair whose expert id lies outside [0, E) is not routed: counts and
    the pair list hold only the valid pairs (stable per expert), the valid
    pairs' rows are within the GEMM tolerance of the oracle, the skipped pairs' rows keep
    their NaN poison, and tokens with only valid pairs sum as usual."""
    E, N, K, T, top_k = 8, 64, 512, 70, 3
    ids = synth.random_ids(1930, T, E, top_k)
    bad = [(3, 1, -1), (10, 0, E), (41, 2, 1 << 20), (69, 2, -7)]
    for t, s_, v in bad:
        ids[t, s_] = v
    Wq, act, rw, Y, Ysum, ws = run_grouped(E, N, K, T, top_k, ids, 1935)
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    counts, offsets, lst = vq.grouped_ws_views(ws, E, T, top_k)
    assert np.array_equal(H.host(counts), np.bincount(flat[valid], minlength=E))
    nvalid = int(valid.sum())
    assert int(H.host(offsets)[E]) == nvalid
    pairs = np.nonzero(valid)[0]
    expect_list = pairs[np.argsort(flat[pairs], kind="stable")]
    assert np.array_equal(H.host(lst)[:nvalid], expect_list)
    ids_ok = np.where(ids >= 0, np.where(ids < E, ids, 0), 0).astype(np.int32)
    Y_ref = oracle.gemm_grouped(oracle.Q4_K, Wq, E, N, K, act, ids_ok, nthreads=8)
    Yh = H.host(Y)
    vmask = valid.reshape(T, top_k)
    H.assert_gemm(oracle.Q4_K, Yh[vmask], Y_ref[vmask], "valid pairs")
    assert np.isnan(Yh[~vmask]).all(), "a skipped pair's row was written"
    full = vmask.all(1)
    H.assert_bitwise(H.host(Ysum)[full], oracle.weighted_sum(Yh[full], rw[full]), "tokens with valid pairs")


def test_grouped_expert_permutation():
    """Permuting expert storage and remapping ids gives the same Y bitwise."""
    E, N, K, T, top_k = 12, 64, 256, 40, 3
    ids = synth.random_ids(1900, T, E, top_k)
    Wq, act, rw, Y, Ysum, ws = run_grouped(E, N, K, T, top_k, ids, 1910)
    perm = np.random.default_rng(1).permutation(E)
    inv = np.argsort(perm)
    Wp = Wq.reshape(E, N, -1)[perm].reshape(E * N, -1)
    ids_p = inv[ids].astype(np.int32)
    H.say("grouped permuted experts")
    Xq = vq.quantize_act(vq.Q8_K, H.to_dev(synth.normal(1911, (T, K))))
    Y2, _, _ = vq.gemm_grouped(vq.Q4_K, H.to_dev(Wp), E, N, K, vq.Q8_K, Xq, T, H.to_dev(ids_p), top_k,
                               route_w=H.to_dev(rw))
    H.assert_bitwise(H.host(Y2), H.host(Y), "permuted experts")


@pytest.mark.parametrize("top_k", [8, 3, 20])
def test_weighted_sum_standalone(top_k):
    """Slot-ordered sum, bit-identical to the oracle, with top_k below, at and
    above the eight slots whose loads the kernel issues up front."""
    T, N = 33, 512
    Y = synth.normal(2000 + top_k, (T, top_k, N))
    w = synth.normal(2001 + top_k, (T, top_k))
    H.say("weighted sum T=%d top_k=%d N=%d" % (T, top_k, N))
    S = vq.weighted_sum(H.to_dev(Y), H.to_dev(w), T, top_k, N)
    H.assert_bitwise(H.host(S), oracle.weighted_sum(Y, w), "weighted sum")
