"""Failure reporting from the device (needs an MI355X).

Kernels never fault or hang on purpose; a bounded wait that gives up, and
(in debug mode) invalid expert ids, are reported through the device error
word.  The conditions are forced from the host: a one-poll bound on the
decode GEMV's loader wait (every kernel still exits normally), and id
tables with an out-of-range and a repeated id.
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


def test_gemv_wait_give_up_is_reported():
    """With the loaders' wait bounded to one poll, the first loader wave of a
    workgroup gives up: its rows come out NaN, vq_device_status reports it
    (and clears it), and with the default bound the same call is exact."""
    N, K = 2560, 9728
    W = synth.normal(2300, (N, K), 0.02)
    x = synth.normal(2301, (K,))
    Wq = oracle.quantize_weights(oracle.Q6_K, W)
    Wd, xd = H.to_dev(Wq), H.to_dev(x)
    vq.device_status()  # nothing pending
    try:
        vq.set_debug(0, wait_polls=1)
        H.say("gemv with a one-poll loader wait N=%d K=%d" % (N, K))
        y = H.host(vq.gemv(vq.Q6_K, Wd, N, K, xd))
    finally:
        vq.set_debug(0, 0)
    assert np.isnan(y).any(), "no workgroup's wait gave up"
    with pytest.raises(vq.VQError) as ei:
        vq.device_status()
    assert ei.value.status == 8 and "loader wait" in str(ei.value)
    vq.device_status()  # cleared
    H.say("gemv with the default bound")
    y = H.host(vq.gemv(vq.Q6_K, Wd, N, K, xd))
    H.assert_bitwise(y, oracle.gemm(oracle.Q6_K, Wq, N, K, oracle.quantize_q8k(x))[0], "gemv after reset")
    vq.device_status()


def test_gemv_wait_give_up_in_sync_mode():
    """In VQ_DEBUG_SYNC mode the call itself returns VQ_ERR_DEVICE."""
    N, K = 9728, 2560
    Wq = oracle.quantize_weights(oracle.Q4_K, synth.normal(2310, (N, K), 0.02))
    Wd, xd = H.to_dev(Wq), H.to_dev(synth.normal(2311, (K,)))
    try:
        vq.set_debug(vq.DEBUG_SYNC, wait_polls=1)
        H.say("gemv, sync mode, one-poll wait")
        with pytest.raises(vq.VQError) as ei:
            vq.gemv(vq.Q4_K, Wd, N, K, xd)
        assert ei.value.status == 8
    finally:
        vq.set_debug(0, 0)
    vq.device_status()


def test_grouped_invalid_ids_reported_in_debug_mode():
    """VQ_DEBUG_CHECK_IDS: an id outside [0, E) and an id repeated within a
    token are reported (bits named in the message); valid tables pass."""
    E, N, K, T, top_k = 8, 64, 256, 40, 3
    Wq = np.concatenate([oracle.quantize_weights(oracle.Q4_K, synth.normal((2320, e), (N, K), 0.02))
                         for e in range(E)])
    Wd = H.to_dev(Wq)
    Xq = vq.quantize_act(vq.Q8_K, H.to_dev(synth.normal(2321, (T, K))))
    ok = synth.random_ids(2322, T, E, top_k)
    try:
        vq.set_debug(vq.DEBUG_SYNC | vq.DEBUG_CHECK_IDS)
        H.say("grouped debug ids: valid table")
        vq.gemm_grouped(vq.Q4_K, Wd, E, N, K, vq.Q8_K, Xq, T, H.to_dev(ok), top_k)
        for what, t, s_, v, needle in (("out of range", 7, 1, E, "outside"), ("repeated", 9, 2, None, "repeated")):
            bad = ok.copy()
            bad[t, s_] = v if v is not None else bad[t, 0]
            H.say("grouped debug ids: %s" % what)
            with pytest.raises(vq.VQError) as ei:
                vq.gemm_grouped(vq.Q4_K, Wd, E, N, K, vq.Q8_K, Xq, T, H.to_dev(bad), top_k)
            assert ei.value.status == 8 and needle in str(ei.value), str(ei.value)
    finally:
        vq.set_debug(0, 0)
    vq.device_status()
