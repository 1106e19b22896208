"""vq_gemm_grouped_noalloc: the grouped call with its routing workspace in the
library's static per-GPU scratch array (needs an MI355X).

Checked through the C ABI against vq_gemm_grouped with a caller workspace:
Y and Ysum bit-identical, on two calls in a row, the second with fewer tokens
and a different routing (the array keeps the first call's contents), and both
against the oracle (Y within the GEMM tolerance, Ysum bitwise).  Sizes beyond
the array are rejected before any launch.
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


def grouped_case(seed, E, N, K, T, top_k):
    Wq = np.concatenate([oracle.quantize_weights(oracle.Q4_K, synth.normal((seed, e), (N, K), 0.02))
                         for e in range(E)])
    X = synth.normal(seed + 1, (T, K))
    ids = synth.random_ids(seed + 2, T, E, top_k)
    logits = synth.normal(seed + 3, (T, top_k))
    z = np.exp(logits - logits.max(1, keepdims=True))
    rw = (z / z.sum(1, keepdims=True)).astype(np.float32)
    return Wq, X, ids, rw


def test_noalloc_matches_workspace_call():
    import torch
    E, N, K, top_k = 16, 80, 512, 4
    for T, seed in ((150, 2100), (37, 2110)):
        Wq, X, ids, rw = grouped_case(seed, E, N, K, T, top_k)
        Wd, idd, rwd = H.to_dev(Wq), H.to_dev(ids), H.to_dev(rw)
        Xq = vq.quantize_act(vq.Q8_K, H.to_dev(X))
        H.say("grouped with workspace E=%d N=%d K=%d T=%d top_k=%d" % (E, N, K, T, top_k))
        Y1, S1, _ = vq.gemm_grouped(vq.Q4_K, Wd, E, N, K, vq.Q8_K, Xq, T, idd, top_k, route_w=rwd,
                                    Y=H.to_dev(np.full((T, top_k, N), np.nan, np.float32)),
                                    Ysum=H.to_dev(np.full((T, N), np.nan, np.float32)))
        Y2 = H.to_dev(np.full((T, top_k, N), np.nan, np.float32))
        S2 = H.to_dev(np.full((T, N), np.nan, np.float32))
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        H.say("grouped no-alloc E=%d N=%d K=%d T=%d top_k=%d" % (E, N, K, T, top_k))
        vq.gemm_grouped_noalloc(vq.Q4_K, Wd, E, N, K, vq.Q8_K, Xq, T, idd, top_k, rwd, Y2, Ysum=S2)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        Y1h, Y2h = H.host(Y1), H.host(Y2)
        H.assert_bitwise(Y2h, Y1h, "no-alloc Y vs workspace call, T=%d" % T)
        H.assert_bitwise(H.host(S2), H.host(S1), "no-alloc Ysum vs workspace call, T=%d" % T)
        Y_ref = oracle.gemm_grouped(oracle.Q4_K, Wq, E, N, K, oracle.quantize_q8k(X), ids, nthreads=8)
        H.assert_close(Y2h, Y_ref, "no-alloc Y vs oracle, T=%d" % T)
        H.assert_bitwise(H.host(S2), oracle.weighted_sum(Y2h, rw), "no-alloc Ysum vs oracle, T=%d" % T)


def test_noalloc_rejects_oversized_routing():
    """More pairs than the static array holds: VQ_ERR_WORKSPACE, no launch."""
    E, top_k = 256, 8
    T = 1 << 17  # 1M pairs
    assert vq.grouped_workspace_bytes(E, T, top_k) > vq.GROUPED_NOALLOC_SCRATCH_BYTES
    fake = 1 << 40
    rc = vq.lib().vq_gemm_grouped_noalloc(vq.Q4_K, fake, E, 64, 256, vq.Q8_K, fake + (1 << 36), T,
                                          fake + (2 << 36), top_k, None, fake + (3 << 36), None, None)
    assert rc == 6  # VQ_ERR_WORKSPACE
    assert b"static" in vq.lib().vq_last_error()
