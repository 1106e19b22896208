"""Pins of the CPU oracle to facts fixed outside the oracle itself.

Runs on the CPU (no GPU marker).  Each test names what pins it: a hand-derived
fixture under tests/golden (with its citation), a library routine (numpy's
binary16 conversion, BLAS fp64, sort/bincount), exact rationals, a closed form
or an invariant of the definition.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import exact, ref_fp64
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _hex32(h):
    return np.array([int(h, 16)], np.uint32).view(np.float32)[0]


# ---------------------------------------------------------------- binary16
def test_f16_decode_matches_numpy_all_patterns():
    bits = np.arange(65536, dtype=np.uint32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_bits_to_f32(int(b)) for b in bits], np.float32)
    same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_f16_encode_matches_numpy_rne():
    rng = np.random.default_rng(0)
    # random float32 bit patterns over the binary16 range and beyond
    xs = [rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32)]
    # exact binary16 midpoints (ties) and their neighbours, incl. subnormals
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    xs += [mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(-np.inf)), -mid]
    xs += [np.array([65504.0, 65519.99, 65520.0, 1e-8, 2.0**-25, 2.0**-25 * 1.0000001, 2.0**-24,
                     0.0, -0.0, np.inf, -np.inf], np.float32)]
    x = np.concatenate(xs)
    ref = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16_bits(float(v)) for v in x], np.uint16)
    nan = np.isnan(x)
    assert (got[~nan] == ref[~nan]).all()
    assert np.isnan(got[nan].view(np.float16)).all()


WTYPES = [oracle.Q4_K, oracle.Q6_K, oracle.Q8_0, oracle.Q5_K]


# ---------------------------------------------------------------- block layouts
def test_q4k_layout_golden():
    g = _load("q4k_block.json")
    q = np.arange(256) % 16
    blk = oracle.q4k_build(g["d16"], g["dmin16"], g["sc"], g["m"], q)
    for k, v in g["bytes_expected"].items():
        assert int(blk[int(k)]) == v, k
    d, dmin, sc, m, qq = oracle.q4k_fields(blk)
    assert (sc == g["sc"]).all() and (m == g["m"]).all() and (qq == q).all()
    assert d == 1.0 and dmin == 0.5
    w = ref_fp64.dequant_weights(oracle.Q4_K, blk[None, :], 1, 256)[0]
    for k, v in g["values_expected"].items():
        assert w[int(k)] == v, k


def test_q6k_layout_golden():
    g = _load("q6k_block.json")
    q = np.arange(256) % 64
    blk = oracle.q6k_build(g["d16"], g["sc"], q)
    for k, v in g["bytes_expected"].items():
        assert int(blk[int(k)]) == v, k
    d, sc, qq = oracle.q6k_fields(blk)
    assert d == 0.5 and (sc == g["sc"]).all() and (qq == q).all()
    w = ref_fp64.dequant_weights(oracle.Q6_K, blk[None, :], 1, 256)[0]
    for k, v in g["values_expected"].items():
        assert w[int(k)] == v, k


def test_q5k_layout_golden():
    g = _load("q5k_block.json")
    q = np.arange(256) % 32
    blk = oracle.q5k_build(g["d16"], g["dmin16"], g["sc"], g["m"], q)
    for k, v in g["bytes_expected"].items():
        assert int(blk[int(k)]) == v, k
    d, dmin, sc, m, qq = oracle.q5k_fields(blk)
    assert (sc == g["sc"]).all() and (m == g["m"]).all() and (qq == q).all()
    assert d == 1.0 and dmin == 0.5
    w = ref_fp64.dequant_weights(oracle.Q5_K, blk[None, :], 1, 256)[0]
    for k, v in g["values_expected"].items():
        assert w[int(k)] == v, k


def test_layout_decoders_agree_on_random_bytes():
    """The C decoder and the independent numpy decoder read the same fields."""
    rng = np.random.default_rng(5)
    for _ in range(50):
        b = rng.integers(0, 256, 144, dtype=np.uint8)
        d, dmin, sc, m, q = oracle.q4k_fields(b)
        d2, dmin2, sc2, m2, q2 = ref_fp64.q4k_decode_fields(b)
        assert (sc == sc2).all() and (m == m2).all() and (q == q2).all()
        assert (np.float32(d) == np.float32(d2)) or (np.isnan(d) and np.isnan(d2))
        b6 = rng.integers(0, 256, 210, dtype=np.uint8)
        d, sc, q = oracle.q6k_fields(b6)
        d2, sc2, q2 = ref_fp64.q6k_decode_fields(b6)
        assert (sc == sc2).all() and (q == q2).all()
        b5 = rng.integers(0, 256, 176, dtype=np.uint8)
        d, dmin, sc, m, q = oracle.q5k_fields(b5)
        d2, dmin2, sc2, m2, q2 = ref_fp64.q5k_decode_fields(b5)
        assert (sc == sc2).all() and (m == m2).all() and (q == q2).all()


# ---------------------------------------------------------------- weight encoders
@pytest.mark.parametrize("wtype", WTYPES)
def test_weight_encoder_roundtrip_bounds(wtype):
    W = synth.normal(7, (64, 1024), 0.02)
    Wq = oracle.quantize_weights(wtype, W)
    Wd = ref_fp64.dequant_weights(wtype, Wq, 64, 1024)
    err = np.abs(W.astype(np.float64) - Wd)
    if wtype == oracle.Q4_K:
        d, dmin, sc, m, q = ref_fp64.q4k_decode_fields(Wq.reshape(64, 4, 144))
        sub = np.arange(256) // 32
        bound = (0.5 * d[..., None] * sc[..., sub] + 7.5 * d[..., None] + 0.5 * dmin[..., None])
    elif wtype == oracle.Q5_K:
        d, dmin, sc, m, q = ref_fp64.q5k_decode_fields(Wq.reshape(64, 4, 176))
        sub = np.arange(256) // 32
        bound = (0.5 * d[..., None] * sc[..., sub] + 15.5 * d[..., None] + 0.5 * dmin[..., None])
    elif wtype == oracle.Q6_K:
        d, sc, q = ref_fp64.q6k_decode_fields(Wq.reshape(64, 4, 210))
        sub = np.arange(256) // 16
        bound = 0.5 * d[..., None] * sc[..., sub] + 15.5 * d[..., None]
    else:
        blocks = Wq.reshape(64, 32, 34)
        d = ref_fp64._f16(blocks[..., 0:2])
        amax = np.abs(W.reshape(64, 32, 32)).max(-1)
        bound = (0.5 * d + 127 * np.abs(amax / 127 - d))[..., None] * np.ones(32)
    assert (err.reshape(bound.shape) <= bound * (1 + 1e-6) + 1e-12).all()
    if wtype in (oracle.Q4_K, oracle.Q5_K, oracle.Q6_K):
        # the quants use the whole range of the format
        assert q.max() == {oracle.Q4_K: 15, oracle.Q5_K: 31, oracle.Q6_K: 63}[wtype]
    # the fit is not degenerate: error well below the signal
    assert np.sqrt(np.mean(err ** 2)) < 0.2 * 0.02


# ---------------------------------------------------------------- Q8_K quantizer
def _build_x(case, n):
    fill = case.get("x_fill", 0.0)
    x = np.full(n, np.nan if fill == "nan" else fill, np.float32)
    for k, v in case["x_nonzero"].items():
        x[int(k)] = _hex32(v) if isinstance(v, str) else v
    return x


def test_q8k_golden():
    g = _load("q8k_quantizer.json")
    for case in g["cases"]:
        x = _build_x(case, 256)
        a = oracle.quantize_q8k(x)
        q = np.full(256, case.get("q_fill", 0), np.int8)
        for k, v in case["q_nonzero"].items():
            q[int(k)] = v
        assert (a.qs[0] == q).all(), case["name"]
        assert a.d.view(np.uint32)[0, 0] == int(case["d_hex"], 16), case["name"]
        assert (a.bsums[0] == case["bsums"]).all(), case["name"]


def test_q8k_invariants():
    X = synth.normal(3, (16, 2048))
    a = oracle.quantize_q8k(X)
    # power-of-two scaling: same bytes, d scaled exactly
    for p in (-3, 5):
        b = oracle.quantize_q8k(X * np.float32(2.0 ** p))
        assert (b.qs == a.qs).all() and (b.bsums == a.bsums).all()
        assert (b.d == a.d * np.float32(2.0 ** p)).all()
    # sign flip: same quants, d negated
    b = oracle.quantize_q8k(-X)
    assert (b.qs == a.qs).all() and (b.bsums == a.bsums).all() and (b.d == -a.d).all()
    # the first max |x| of every super-block quantizes to -127 and fixes sign(d) = -sign(mx)
    Xb = X.reshape(16, 8, 256)
    first = np.abs(Xb).argmax(-1)
    qb = a.qs.reshape(16, 8, 256)
    assert (np.take_along_axis(qb, first[..., None], -1) == -127).all()
    mx = np.take_along_axis(Xb, first[..., None], -1)[..., 0]
    assert (np.sign(a.d) == -np.sign(mx)).all()
    # round trip |x - d q| <= |d|/2 (1 + 2^-20)
    deq = a.d[:, :, None].astype(np.float64) * qb
    assert (np.abs(Xb - deq) <= 0.5 * np.abs(a.d[:, :, None]) * (1 + 2.0 ** -20)).all()
    # bsums are the 16-element sums of the quants
    assert (a.bsums == a.qs.reshape(16, 128, 16).astype(np.int32).sum(-1)).all()


# ---------------------------------------------------------------- Q8_1 quantizer
def test_q8_1_golden():
    g = _load("q8_1_quantizer.json")
    for case in g["cases"]:
        x = _build_x(case, 32)
        a = oracle.quantize_q8_1(x)
        q = np.zeros(32, np.int8)
        for k, v in case["q_nonzero"].items():
            q[int(k)] = v
        assert (a.qs[0] == q).all(), case["name"]
        assert int(a.d[0, 0]) == int(case["d16_hex"], 16), case["name"]
        assert int(a.s[0, 0]) == int(case["s16_hex"], 16), case["name"]


def test_q8_1_invariants():
    X = synth.normal(4, (8, 1024))
    a = oracle.quantize_q8_1(X)
    Xb = X.reshape(8, 32, 32).astype(np.float64)
    qb = a.qs.reshape(8, 32, 32)
    amax = np.abs(Xb).max(-1)
    d32 = (amax / 127).astype(np.float32).astype(np.float64)
    # |x - d q| <= d/2 (1 + eps) with the binary32 d used for q
    assert (np.abs(Xb - d32[..., None] * qb) <= 0.5 * d32[..., None] * (1 + 2.0 ** -20)).all()
    # stored d is binary16(amax/127)
    assert (a.d == (amax / 127).astype(np.float32).astype(np.float16).view(np.uint16)).all()
    # the stored block sum is within binary16 rounding of the exact sum
    s = a.s.view(np.float16).astype(np.float64)
    exact_sum = Xb.sum(-1)
    assert (np.abs(s - exact_sum) <= np.abs(exact_sum) * 2.0 ** -10 + 1e-5).all()
    # the element of largest |x| maps to +-127
    first = np.abs(Xb).argmax(-1)
    assert (np.abs(np.take_along_axis(qb, first[..., None], -1)) == 127).all()


# ---------------------------------------------------------------- dots
def _case(wtype, M, N, K, seed):
    W = synth.normal(seed, (N, K), 0.02)
    X = synth.normal(seed + 1, (M, K))
    Wq = oracle.quantize_weights(wtype, W)
    act = oracle.quantize_q8_1(X) if wtype == oracle.Q8_0 else oracle.quantize_q8k(X)
    return Wq, act


@pytest.mark.parametrize("wtype", WTYPES)
def test_oracle_gemm_vs_fp64_definition(wtype):
    Wq, act = _case(wtype, 8, 96, 2048, 100 + wtype)
    y = oracle.gemm(wtype, Wq, 96, 2048, act)
    r = ref_fp64.gemm_fp64(wtype, Wq, 96, 2048, act)
    floored, _ = ref_fp64.max_rel_err(y, r)
    assert floored <= 2e-5
    assert ref_fp64.nmse(y, r) <= 1e-11


@pytest.mark.parametrize("wtype", WTYPES)
def test_oracle_gemm_vs_exact_rationals(wtype):
    K = 512 if wtype != oracle.Q8_0 else 128
    Wq, act = _case(wtype, 2, 3, K, 200 + wtype)
    y = oracle.gemm(wtype, Wq, 3, K, act)
    ex = exact.gemm_exact(wtype, Wq, 3, K, act)
    A = ref_fp64.dequant_act(act)
    Wd = ref_fp64.dequant_weights(wtype, Wq, 3, K)
    scale = np.abs(A) @ np.abs(Wd).T  # sum |terms|: fp32 error bound scale
    for m in range(2):
        for n in range(3):
            err = abs(float(y[m, n]) - float(ex[m][n]))
            assert err <= 1e-6 * scale[m, n] + 1e-30, (m, n, err, scale[m, n])


@pytest.mark.parametrize("wtype", WTYPES)
def test_random_byte_blocks_vs_definitions(wtype):
    """Random-byte fuzz: random sc/m/q bytes, binary16 d in [2^-10, 1]."""
    rng = np.random.default_rng(300 + wtype)
    N, K, M = 5, 512, 3
    bb = oracle.BLOCK_BYTES[wtype]
    nb = K // oracle.BLOCK_ELEMS[wtype]
    Wq = rng.integers(0, 256, (N, nb, bb), dtype=np.uint8)
    dvals = (2.0 ** rng.uniform(-10, 0, (N, nb, 2))).astype(np.float16).view(np.uint8)
    dvals = dvals.reshape(N, nb, 4)
    if wtype in (oracle.Q4_K, oracle.Q5_K):
        Wq[..., 0:4] = dvals
    elif wtype == oracle.Q6_K:
        Wq[..., 208:210] = dvals[..., 0:2]
    else:
        Wq[..., 0:2] = dvals[..., 0:2]
    Wq = Wq.reshape(N, nb * bb)
    X = synth.normal(400 + wtype, (M, K))
    act = oracle.quantize_q8_1(X) if wtype == oracle.Q8_0 else oracle.quantize_q8k(X)
    y = oracle.gemm(wtype, Wq, N, K, act)
    r = ref_fp64.gemm_fp64(wtype, Wq, N, K, act)
    A = ref_fp64.dequant_act(act)
    Wd = ref_fp64.dequant_weights(wtype, Wq, N, K)
    scale = np.abs(A) @ np.abs(Wd).T
    assert (np.abs(y - r) <= 1e-6 * scale).all()
    ex = exact.gemm_exact(wtype, Wq[:2], 2, K, oracle.Q81(act.qs[:1], act.d[:1], act.s[:1])
                          if wtype == oracle.Q8_0 else oracle.Q8K(act.qs[:1], act.d[:1], act.bsums[:1]))
    for n in range(2):
        assert abs(float(r[0, n]) - float(ex[0][n])) <= 1e-12 * scale[0, n]


def test_unit_scale_probes_give_exact_subblock_sums():
    """d=1, dmin=0, one sc_j=1 and activations with iscale=1: y equals I_j."""
    a = ((np.arange(256) * 37) % 255 - 127).astype(np.float32)  # a[0] = -127 is the first max
    act = oracle.quantize_q8k(a)
    assert act.d[0, 0] == 1.0 and (act.qs[0] == a.astype(np.int8)).all()
    rng = np.random.default_rng(9)
    q = rng.integers(0, 16, 256)
    for j in range(8):
        sc = np.zeros(8, np.int32)
        sc[j] = 1
        blk = oracle.q4k_build(0x3C00, 0, sc, np.zeros(8, np.int32), q)
        y = oracle.gemm(oracle.Q4_K, blk[None, :], 1, 256, act)[0, 0]
        I_brute = int(sum(int(q[i]) * int(a[i]) for i in range(32 * j, 32 * j + 32)))
        assert y == I_brute
        assert oracle.subblock_sums(oracle.Q4_K, blk, act.qs[0])[j] == I_brute
    q5 = rng.integers(0, 32, 256)
    for j in range(8):
        sc = np.zeros(8, np.int32)
        sc[j] = 1
        blk = oracle.q5k_build(0x3C00, 0, sc, np.zeros(8, np.int32), q5)
        y = oracle.gemm(oracle.Q5_K, blk[None, :], 1, 256, act)[0, 0]
        I_brute = int(sum(int(q5[i]) * int(a[i]) for i in range(32 * j, 32 * j + 32)))
        assert y == I_brute
        assert oracle.subblock_sums(oracle.Q5_K, blk, act.qs[0])[j] == I_brute
    q6 = rng.integers(0, 64, 256)
    for j in range(16):
        sc = np.zeros(16, np.int32)
        sc[j] = 1
        blk = oracle.q6k_build(0x3C00, sc, q6)
        y = oracle.gemm(oracle.Q6_K, blk[None, :], 1, 256, act)[0, 0]
        I_brute = int(sum((int(q6[i]) - 32) * int(a[i]) for i in range(16 * j, 16 * j + 16)))
        assert y == I_brute


def test_closed_forms():
    Wq, act = _case(oracle.Q4_K, 4, 16, 1024, 500)
    # X = 0 -> Y = 0
    z = oracle.quantize_q8k(np.zeros((4, 1024), np.float32))
    assert (oracle.gemm(oracle.Q4_K, Wq, 16, 1024, z) == 0).all()
    # d = dmin = 0 -> Y = 0
    W0 = Wq.reshape(16, 4, 144).copy()
    W0[..., 0:4] = 0
    assert (oracle.gemm(oracle.Q4_K, W0.reshape(16, -1), 16, 1024, act) == 0).all()
    # Q6_K with every q = 32 -> Y = 0
    blk = oracle.q6k_build(0x3C00, np.arange(16) - 8, np.full(256, 32))
    a6 = oracle.quantize_q8k(synth.normal(501, (3, 256)))
    assert (oracle.gemm(oracle.Q6_K, blk[None, :], 1, 256, a6) == 0).all()
    # Q4_K with every q = 0 isolates the min term: y = -sum_b da*dmin*sum_j m_j*bsum32_j
    blk = oracle.q4k_build(0x3C00, 0x3800, np.arange(8) + 1, np.arange(8) * 7 + 3, np.zeros(256))
    y = oracle.gemm(oracle.Q4_K, blk[None, :], 1, 256, a6)
    xd = ref_fp64.dequant_act(a6)
    mvec = np.repeat(np.arange(8) * 7 + 3, 32) * 0.5
    assert np.allclose(y[:, 0], -(xd @ mvec), rtol=1e-6, atol=0)
    # permuting the rows of W permutes the columns of Y bitwise
    perm = np.random.default_rng(1).permutation(16)
    y = oracle.gemm(oracle.Q4_K, Wq, 16, 1024, act)
    yp = oracle.gemm(oracle.Q4_K, Wq[perm], 16, 1024, act)
    assert (yp == y[:, perm]).all()


def test_threads_do_not_change_results():
    Wq, act = _case(oracle.Q6_K, 7, 33, 512, 600)
    assert (oracle.gemm(oracle.Q6_K, Wq, 33, 512, act, nthreads=1)
            == oracle.gemm(oracle.Q6_K, Wq, 33, 512, act, nthreads=4)).all()


# ---------------------------------------------------------------- routing, expert sum
def test_route_golden_and_library_sort():
    g = _load("routing.json")
    counts, offsets, lst = oracle.route(np.array(g["ids"], np.int32), g["E"])
    assert counts.tolist() == g["counts"] and offsets.tolist() == g["offsets"]
    assert lst.tolist() == g["list"]
    ids = synth.random_ids(11, 300, 64, 8)
    counts, offsets, lst = oracle.route(ids, 64)
    flat = ids.reshape(-1)
    assert (counts == np.bincount(flat, minlength=64)).all()
    assert (lst == np.argsort(flat, kind="stable")).all()
    assert offsets[-1] == flat.size and (np.diff(offsets) == counts).all()


@pytest.mark.parametrize("wtype", WTYPES)
def test_grouped_matches_dense_per_expert(wtype):
    """Broadcast arm: each slot is its expert's dense product with the token row."""
    E, N, K, T, top_k = 6, 24, 512, 10, 3
    W = np.stack([synth.normal((700, e), (N, K), 0.02) for e in range(E)])
    Wq = np.stack([oracle.quantize_weights(wtype, W[e]) for e in range(E)])
    X = synth.normal(701, (T, K))
    act = oracle.quantize_q8_1(X) if wtype == oracle.Q8_0 else oracle.quantize_q8k(X)
    ids = synth.random_ids(702, T, E, top_k)
    Y = oracle.gemm_grouped(wtype, Wq.reshape(E * N, -1), E, N, K, act, ids)
    for e in range(E):
        dense = oracle.gemm(wtype, Wq[e], N, K, act)
        t, s = np.nonzero(ids == e)
        assert (Y[t, s] == dense[t]).all()
    # against the fp64 definition, slot by slot
    r64 = np.stack([ref_fp64.gemm_fp64(wtype, Wq[ids[t, s]], N, K,
                                       oracle.quantize_q8_1(X[t:t + 1]) if wtype == oracle.Q8_0
                                       else oracle.quantize_q8k(X[t:t + 1]))[0]
                    for t in range(T) for s in range(top_k)]).reshape(T, top_k, N)
    assert ref_fp64.max_rel_err(Y, r64)[0] <= 5e-4


@pytest.mark.parametrize("wtype", WTYPES)
def test_grouped_per_row_arm(wtype):
    """Per-row arm: each pair has its own activation row.  With every pair's
    row equal to its token's row it reduces to the broadcast arm bitwise; with
    distinct rows each slot is its expert's dense product with that row."""
    E, N, K, T, top_k = 5, 16, 256, 7, 2
    W = np.stack([synth.normal((710, e), (N, K), 0.02) for e in range(E)])
    Wq = np.stack([oracle.quantize_weights(wtype, W[e]) for e in range(E)]).reshape(E * N, -1)
    ids = synth.random_ids(712, T, E, top_k)
    q = oracle.quantize_q8_1 if wtype == oracle.Q8_0 else oracle.quantize_q8k
    X = synth.normal(711, (T, K))
    Xrep = np.repeat(X, top_k, axis=0)
    Yb = oracle.gemm_grouped(wtype, Wq, E, N, K, q(X), ids)
    Yr = oracle.gemm_grouped(wtype, Wq, E, N, K, q(Xrep), ids, per_row=True)
    assert (Yb.view(np.uint32) == Yr.view(np.uint32)).all()
    Xp = synth.normal(713, (T * top_k, K))
    Yp = oracle.gemm_grouped(wtype, Wq, E, N, K, q(Xp), ids, per_row=True)
    Wr = Wq.reshape(E, N, -1)
    for t in range(T):
        for s in range(top_k):
            dense = oracle.gemm(wtype, Wr[ids[t, s]], N, K, q(Xp[t * top_k + s:t * top_k + s + 1]))[0]
            assert (Yp[t, s].view(np.uint32) == dense.view(np.uint32)).all()


def test_weighted_sum_golden():
    g = _load("weighted_sum.json")
    for case in g["cases"]:
        Y = np.array(case["y"], np.float32).reshape(1, -1, 1)
        w = np.array(case["w"], np.float32).reshape(1, -1)
        out = oracle.weighted_sum(Y, w)
        assert out[0, 0] == np.float32(case["ysum"]), case["name"]
    # one-hot weights select a slot exactly
    Y = synth.normal(800, (5, 8, 16))
    w = np.zeros((5, 8), np.float32)
    w[np.arange(5), np.arange(5) % 8] = 1.0
    out = oracle.weighted_sum(Y, w)
    assert (out == Y[np.arange(5), np.arange(5) % 8]).all()


# ---------------------------------------------------------------- workloads
def test_workload_shapes_and_routing():
    ids, w = synth.routing(T=64, E=256, top_k=8)
    assert ids.shape == (64, 8) and w.shape == (64, 8)
    assert all(len(set(r)) == 8 for r in ids.tolist())
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)
    cols = synth.outlier_columns(2560)
    assert cols.size == 26 and np.unique(cols).size == 26
    assert synth.outlier_columns(9728).size == 97


# ------------------------------------------------------------------ producers
def test_rmsnorm_pins():
    """RMSNorm pins from the mathematics: a worked example, unit output RMS,
    scale invariance, eps inside the root, gamma per position."""
    # [3, 4]: mean of squares 12.5 = 25/2, so x / rms = x * sqrt(2) / 5
    y = oracle.rmsnorm(np.array([[3.0, 4.0]], np.float32), np.array([1.0, 2.0], np.float32), 0.0)
    assert np.allclose(y, [[3 * np.sqrt(2) / 5, 8 * np.sqrt(2) / 5]], rtol=1e-15, atol=0)
    X = synth.normal(3100, (5, 768))
    ones = np.ones(768, np.float32)
    y = oracle.rmsnorm(X, ones, 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-12, atol=0)
    assert np.allclose(oracle.rmsnorm(X * np.float32(8.0), ones, 0.0), y, rtol=1e-13, atol=0)
    # constant rows c with eps: c / sqrt(c^2 + eps); c = 1, eps = 3 -> 1/2
    g = np.arange(1, 257, dtype=np.float32)
    y = oracle.rmsnorm(np.ones((2, 256), np.float32), g, 3.0)
    assert np.array_equal(y, np.stack([g.astype(np.float64) / 2] * 2))
    # zero row: zero output for any eps > 0
    assert not oracle.rmsnorm(np.zeros((1, 256), np.float32), g, 1e-6).any()


def test_silu_mul_pins():
    """SiLU-mul pins: sigmoid(ln 3) = 3/4, the odd part silu(x) - silu(-x) = x,
    the even part silu(x) + silu(-x) = x tanh(x/2), linearity in up."""
    l3 = np.float32(np.log(3.0))
    y = oracle.silu_mul(np.array([[0.0, l3, -l3]], np.float32), np.ones((1, 3), np.float32))
    assert y[0, 0] == 0.0
    assert abs(y[0, 1] - 0.75 * float(l3)) <= 1e-7 * float(l3)
    assert abs(y[0, 2] + 0.25 * float(l3)) <= 1e-7 * float(l3)
    x = synth.normal(3101, (3, 512), 4.0)
    ones = np.ones_like(x)
    p, n = oracle.silu_mul(x, ones), oracle.silu_mul(-x, ones)
    xd = x.astype(np.float64)
    assert np.allclose(p - n, xd, rtol=1e-12, atol=1e-12)
    assert np.allclose(p + n, xd * np.tanh(xd / 2), rtol=1e-10, atol=1e-12)
    u = synth.normal(3102, (3, 512))
    assert np.allclose(oracle.silu_mul(x, u), p * u.astype(np.float64), rtol=1e-15, atol=0)
