"""C-ABI boundary checks that need no GPU.

The library loads, exports every function include/vq.h declares, reports the
documented sizes, and rejects bad arguments on the host -- before any launch --
with a status and a message naming the offending type or size.  Only calls
that fail validation (or are empty) are made here, so nothing reaches the GPU.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vq.h")


@pytest.fixture(scope="module")
def vq():
    import block_quantized_matmul_fp32_amd as m
    if not os.path.exists(m.LIB_PATH):
        from block_quantized_matmul_fp32_amd import build
        build.build()
    m.lib()
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(vq_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_expected_api():
    names = declared_functions()
    for f in ("vq_quantize_act", "vq_gemv", "vq_gemm", "vq_gemm_grouped", "vq_gemm_grouped_rows",
              "vq_is_supported", "vq_weighted_sum", "vq_quantize_weights"):
        assert f in names


def test_library_exports_every_declared_symbol(vq):
    L = vq.lib()
    missing = [f for f in declared_functions() if not hasattr(L, f)]
    assert not missing, missing
    out = subprocess.run(["nm", "-D", "--defined-only", vq.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (vq_[a-z0-9_]+)", out))
    assert set(declared_functions()) <= exported
    assert set(vq.EXPORTS) == set(declared_functions())


def test_sizes(vq):
    assert vq.block_bytes(vq.Q4_K) == 144 and vq.block_bytes(vq.Q6_K) == 210
    assert vq.block_bytes(vq.Q8_0) == 34 and vq.block_values(vq.Q8_0) == 32
    assert vq.weight_bytes(vq.Q4_K, 9728, 2560) == 9728 * 10 * 144
    assert vq.weight_bytes(vq.Q6_K, 2560, 9728) == 2560 * 38 * 210
    assert vq.weight_bytes(vq.Q8_0, 4096, 2048) == 4096 * 64 * 34
    assert vq.weight_bytes(vq.Q4_K, 10, 100) == 0
    a = lambda x: (x + 255) // 256 * 256
    M, K = 3, 512
    assert vq.act_d_offset(vq.Q8_K, M, K) == a(M * K)
    assert vq.act_aux_offset(vq.Q8_K, M, K) == a(M * K) + a(M * 2 * 4)
    assert vq.act_bytes(vq.Q8_K, M, K) == a(M * K) + a(M * 2 * 4) + a(M * 32 * 2)
    K = 96
    assert vq.act_aux_offset(vq.Q8_1, M, K) == a(M * K) + a(M * 3 * 2)
    assert vq.act_bytes(vq.Q8_1, M, K) == a(M * K) + 2 * a(M * 3 * 2)
    assert vq.act_bytes(vq.Q8_K, 1, 100) == 0


def test_capability_query(vq):
    S = vq.is_supported
    for op in (vq.OP_GEMV, vq.OP_GEMM, vq.OP_GEMM_GROUPED):
        assert S(vq.Q4_K, vq.Q8_K, op) and S(vq.Q6_K, vq.Q8_K, op) and S(vq.Q8_0, vq.Q8_1, op)
        assert not S(vq.Q4_K, vq.Q8_1, op) and not S(vq.Q8_0, vq.Q8_K, op)
        assert not S(vq.Q8_K, vq.Q8_K, op) and not S(17, vq.Q8_K, op)
    assert not S(vq.Q4_K, vq.Q8_K, 7)


FAKE = 0x10000000  # never dereferenced: every call below fails validation first


def _err(vq, status, fn, *args):
    r = getattr(vq.lib(), fn)(*args)
    msg = vq.lib().vq_last_error().decode()
    assert r == status, (vq.STATUS.get(r), msg)
    return msg


def test_unsupported_types_are_named(vq):
    msg = _err(vq, 2, "vq_gemm", 9, FAKE, 64, 256, vq.Q8_K, FAKE, 4, FAKE, 64, None, 0, None)
    assert "unknown" in msg and "9" in msg
    msg = _err(vq, 2, "vq_gemv", vq.Q8_K, FAKE, 64, 256, FAKE, FAKE, None, None)
    assert "Q8_K" in msg
    msg = _err(vq, 2, "vq_quantize_act", vq.Q4_K, FAKE, 4, 256, 256, FAKE, None)
    assert "Q4_K" in msg
    for fn in ("vq_gemm_grouped", "vq_gemm_grouped_rows"):
        msg = _err(vq, 2, fn, vq.Q8_1, FAKE, 8, 64, 256, vq.Q8_K, FAKE, 4, FAKE, 2, FAKE,
                   FAKE, None, FAKE, 1 << 20, None)
        assert "Q8_1" in msg and fn in msg
    _err(vq, 3, "vq_gemm_grouped_rows", vq.Q8_0, FAKE, 8, 64, 256, vq.Q8_K, FAKE, 4, FAKE, 2, FAKE,
         FAKE, None, FAKE, 1 << 20, None)


def test_type_pairing(vq):
    msg = _err(vq, 3, "vq_gemm", vq.Q8_0, FAKE, 64, 256, vq.Q8_K, FAKE, 4, FAKE, 64, None, 0, None)
    assert "Q8_0" in msg and "Q8_1" in msg
    _err(vq, 3, "vq_gemm", vq.Q6_K, FAKE, 64, 256, vq.Q8_1, FAKE, 4, FAKE, 64, None, 0, None)


def test_shape_errors(vq):
    msg = _err(vq, 4, "vq_gemm", vq.Q4_K, FAKE, 64, 300, vq.Q8_K, FAKE, 4, FAKE, 64, None, 0, None)
    assert "300" in msg and "256" in msg
    _err(vq, 4, "vq_gemm", vq.Q8_0, FAKE, 64, 48, vq.Q8_1, FAKE, 4, FAKE, 64, None, 0, None)
    _err(vq, 4, "vq_gemm", vq.Q4_K, FAKE, -1, 256, vq.Q8_K, FAKE, 4, FAKE, 64, None, 0, None)
    _err(vq, 4, "vq_gemm", vq.Q4_K, FAKE, 64, 256, vq.Q8_K, FAKE, 4, FAKE, 10, None, 0, None)  # ldy < N
    _err(vq, 4, "vq_quantize_act", vq.Q8_K, FAKE, 4, 256, 100, FAKE, None)          # ldx < K
    _err(vq, 4, "vq_gemm_grouped", vq.Q4_K, FAKE, 2000, 64, 256, vq.Q8_K, FAKE, 4, FAKE, 2, FAKE,
         FAKE, None, FAKE, 1 << 20, None)  # E > 1024
    _err(vq, 4, "vq_gemm_grouped", vq.Q4_K, FAKE, 8, 60, 256, vq.Q8_K, FAKE, 4, FAKE, 2, FAKE,
         FAKE, None, FAKE, 1 << 20, None)  # N % 16
    _err(vq, 4, "vq_weighted_sum", FAKE, FAKE, 4, 2, 10, FAKE, None)                 # N % 4


def test_null_misaligned_alias_workspace(vq):
    _err(vq, 1, "vq_gemm", vq.Q4_K, None, 64, 256, vq.Q8_K, FAKE, 4, FAKE, 64, None, 0, None)
    _err(vq, 1, "vq_gemm", vq.Q4_K, FAKE + 2, 64, 256, vq.Q8_K, FAKE + 0x100000, 4, FAKE + 0x200000, 64, None, 0, None)
    # Y overlapping W
    msg = _err(vq, 5, "vq_gemm", vq.Q4_K, FAKE, 64, 256, vq.Q8_K, FAKE + 0x100000, 4, FAKE + 64, 64, None, 0, None)
    assert "overlap" in msg
    # y overlapping x in the GEMV
    _err(vq, 5, "vq_gemv", vq.Q4_K, FAKE, 64, 256, FAKE + 0x100000, FAKE + 0x100000 + 16, None, None)
    # Xq overlapping X
    _err(vq, 5, "vq_quantize_act", vq.Q8_K, FAKE, 4, 256, 256, FAKE + 256, None)
    need = vq.grouped_workspace_bytes(8, 4, 2)
    msg = _err(vq, 6, "vq_gemm_grouped", vq.Q4_K, FAKE, 8, 64, 256, vq.Q8_K, FAKE + 0x100000, 4,
               FAKE + 0x200000, 2, FAKE + 0x300000, FAKE + 0x400000, None, FAKE + 0x500000, need - 1, None)
    assert str(need) in msg
    # Ysum without route_w
    _err(vq, 1, "vq_gemm_grouped", vq.Q4_K, FAKE, 8, 64, 256, vq.Q8_K, FAKE + 0x100000, 4,
         FAKE + 0x200000, 2, None, FAKE + 0x400000, FAKE + 0x480000, FAKE + 0x500000, need, None)


def test_gemm_workspace_checks(vq):
    """vq_gemm's workspace: 256-byte alignment and no overlap with W, Xq or Y,
    checked before any launch; vq_gemm_workspace sizes (none for Q8_0 or the
    GEMV-kernel batches; the split plan's parts per grid size; the cap)."""
    base = dict(W=FAKE, Xq=FAKE + 0x4000000, Y=FAKE + 0x8000000)
    args = lambda ws, wsb: (vq.Q6_K, base["W"], 640, 4096, vq.Q8_K, base["Xq"], 256, base["Y"], 640, ws, wsb,
                            None)
    msg = _err(vq, 1, "vq_gemm", *args(FAKE + 0xC000000 + 16, 1 << 20))
    assert "256-byte" in msg
    msg = _err(vq, 5, "vq_gemm", *args(base["Xq"] + 0x100, 1 << 20))
    assert "workspace" in msg
    _err(vq, 5, "vq_gemm", *args(base["W"], 1 << 20))
    _err(vq, 5, "vq_gemm", *args(base["Y"] - 0x100, 1 << 20))
    assert vq.gemm_workspace(vq.Q8_0, 2048, 4096, 2048) == 0
    assert vq.gemm_workspace(vq.Q4_K, 1, 9728, 2560) == 0          # GEMV-kernel arm
    assert vq.gemm_workspace(vq.Q4_K, 2048, 9728, 2560) == 0       # 1216 tiles fill the chip: no split
    assert vq.gemm_workspace(vq.Q6_K, 512, 2560, 9728) == 65536 + 80 * 6 * 128 * 128 * 4   # two per CU
    # 320 tiles: three parts fill 1.875 rounds of two workgroups per CU, two parts 1.25
    assert vq.gemm_workspace(vq.Q6_K, 2048, 2560, 9728) == 65536 + 320 * 3 * 128 * 128 * 4
    assert vq.gemm_workspace(vq.Q6_K, 3200, 2560, 9728) == 65536 + 500 * 2 * 128 * 128 * 4  # ties go to two
    assert vq.gemm_workspace(vq.Q4_K, 512, 9728, 2560) == 0         # 304 tiles, 10 steps: no split
    assert vq.gemm_workspace(vq.Q4_K, 200, 9728, 2560) == 65536 + 152 * 3 * 128 * 128 * 4  # two per CU
    assert vq.gemm_workspace(vq.Q4_K, 64, 9728, 2560) == 65536 + 76 * 3 * 128 * 128 * 4   # parts of 3+ steps
    assert vq.gemm_workspace(vq.Q6_K, 200, 2560, 9728) == 65536 + 40 * 6 * 128 * 128 * 4  # 8 is not twice 6
    small = vq.gemm_workspace(vq.Q6_K, 256, 640, 4096)             # 10 tiles, 16 steps: split K
    assert small > 0 and small % 256 == 0
    assert vq.gemm_workspace(vq.Q4_K, 0, 640, 4096) == 0
    assert vq.gemm_workspace(vq.Q4_K, 256, 640, 1000) == 0         # K not a multiple of 256
    assert vq.gemm_workspace(9, 256, 640, 4096) == 0


def test_overrides_are_per_thread(vq):
    """The crossover and row-block overrides apply to the calling thread only."""
    import threading
    seen = {}
    L = vq.lib()
    assert L.vq_set_small_batch_max(vq.Q4_K, 3) == 0
    try:
        t = threading.Thread(target=lambda: seen.setdefault("other", L.vq_small_batch_max(vq.Q4_K)))
        t.start()
        t.join()
        assert L.vq_small_batch_max(vq.Q4_K) == 3
        assert seen["other"] == 8
        # a row-block cap on another thread leaves this thread's workspace plan alone
        before = vq.gemm_workspace(vq.Q6_K, 1000, 640, 4096)
        t = threading.Thread(target=lambda: L.vq_set_gemm_row_block(128))
        t.start()
        t.join()
        assert vq.gemm_workspace(vq.Q6_K, 1000, 640, 4096) == before
    finally:
        L.vq_set_small_batch_max(vq.Q4_K, -1)


def test_grouped_noalloc_rejects_oversized_routing(vq):
    """The static-scratch grouped call rejects a routing workspace larger than
    its array before any launch (and before it looks up the array)."""
    assert vq.grouped_workspace_bytes(256, 1 << 17, 8) > vq.GROUPED_NOALLOC_SCRATCH_BYTES
    msg = _err(vq, 6, "vq_gemm_grouped_noalloc", vq.Q4_K, FAKE, 256, 64, 256, vq.Q8_K, FAKE + 0x100000, 1 << 17,
               FAKE + 0x200000, 8, None, FAKE + 0x300000, None, None)
    assert "static" in msg and str(vq.GROUPED_NOALLOC_SCRATCH_BYTES) in msg


def test_stream_probe_checks(vq):
    """vq_stream_probe validates like vq_gemv, and its sink's size and aliasing."""
    _err(vq, 2, "vq_stream_probe", 9, FAKE, 64, 256, FAKE + 0x100000, 256, None)
    _err(vq, 4, "vq_stream_probe", vq.Q4_K, FAKE, 64, 300, FAKE + 0x100000, 256, None)
    msg = _err(vq, 6, "vq_stream_probe", vq.Q4_K, FAKE, 64, 256, FAKE + 0x100000, 255, None)
    assert "256" in msg
    _err(vq, 5, "vq_stream_probe", vq.Q4_K, FAKE, 64, 256, FAKE + 64, 256, None)
    _err(vq, 1, "vq_stream_probe", vq.Q4_K, FAKE + 4, 64, 256, FAKE + 0x100000, 256, None)
    assert vq.lib().vq_stream_probe(vq.Q4_K, None, 0, 256, None, 0, None) == 0


def test_mfma_probe_checks(vq):
    """vq_mfma_probe: the round count's range and the sink (host only)."""
    _err(vq, 1, "vq_mfma_probe", 0, FAKE, 4, None, None)
    _err(vq, 1, "vq_mfma_probe", (1 << 24) + 1, FAKE, 4, None, None)
    _err(vq, 1, "vq_mfma_probe", 16, None, 4, None, None)
    _err(vq, 1, "vq_mfma_probe", 16, FAKE + 2, 4, None, None)
    msg = _err(vq, 6, "vq_mfma_probe", 16, FAKE, 3, None, None)
    assert "4" in msg


def test_set_debug_checks(vq):
    """vq_set_debug: unknown flags and out-of-range bounds are rejected (host only)."""
    _err(vq, 1, "vq_set_debug", 8, 0)
    _err(vq, 1, "vq_set_debug", 0, -1)
    assert vq.lib().vq_set_debug(vq.DEBUG_SYNC | vq.DEBUG_CHECK_IDS, 5) == 0
    assert vq.lib().vq_set_debug(0, 0) == 0
    assert vq.lib().vq_status_string(8) == b"VQ_ERR_DEVICE"


def test_empty_calls_are_ok(vq):
    L = vq.lib()
    assert L.vq_gemm(vq.Q4_K, None, 0, 256, vq.Q8_K, None, 0, None, 0, None, 0, None) == 0
    assert L.vq_quantize_act(vq.Q8_1, None, 0, 64, 64, None, None) == 0
    assert L.vq_gemv(vq.Q6_K, None, 0, 256, None, None, None, None) == 0


def test_status_strings_and_stats(vq):
    L = vq.lib()
    assert L.vq_status_string(4) == b"VQ_ERR_SHAPE"
    vq.reset_stats()
    st = vq.get_stats()
    assert set(st) == set(vq.STAT_FIELDS) and all(v == 0 for v in st.values())


def test_small_batch_crossover_setting(vq):
    """vq_set_small_batch_max: defaults, range and type checks (host only)."""
    defaults = {vq.Q4_K: 8, vq.Q6_K: 8, vq.Q8_0: 32, vq.Q5_K: 8}
    for w, d in defaults.items():
        assert vq.small_batch_max(w) == d
    try:
        vq.set_small_batch_max(vq.Q6_K, 3)
        assert vq.small_batch_max(vq.Q6_K) == 3
        vq.set_small_batch_max(vq.Q6_K, -1)
        assert vq.small_batch_max(vq.Q6_K) == 8
        with pytest.raises(vq.VQError, match="INVALID_ARG"):
            vq.set_small_batch_max(vq.Q4_K, 65)
        with pytest.raises(vq.VQError, match="INVALID_ARG"):
            vq.set_small_batch_max(vq.Q4_K, -2)
        with pytest.raises(vq.VQError, match="UNSUPPORTED_TYPE"):
            vq.set_small_batch_max(vq.Q8_K, 4)
        assert vq.small_batch_max(vq.Q8_K) == -1
    finally:
        for w in defaults:
            vq.set_small_batch_max(w, -1)


def test_gemm_row_block_setting(vq):
    """vq_set_gemm_row_block: 0 and positive caps accepted, negative rejected
    (host only; the blocked launches are checked against one launch on the GPU)."""
    try:
        vq.set_gemm_row_block(200)
        vq.set_gemm_row_block(0)
        with pytest.raises(vq.VQError, match="INVALID_ARG"):
            vq.set_gemm_row_block(-1)
    finally:
        vq.set_gemm_row_block(0)


def test_gemv_rejects_rows_too_long_for_lds(vq):
    """The fused GEMV keeps a weight row and the quantized activation in LDS:
    K past that limit is a shape error, checked on the host before any
    pointer is looked at (no GPU needed)."""
    L = vq.lib()
    assert L.vq_gemv(vq.Q8_0, None, 1, 65536, None, None, None, None) == 4  # VQ_ERR_SHAPE
    assert L.vq_gemv(vq.Q4_K, None, 1, 65536, None, None, None, None) == 1  # fits: then the null pointers
    assert L.vq_gemv(vq.Q6_K, None, 1, 1 << 17, None, None, None, None) == 4


def test_binding_rejects_host_short_and_strided_buffers(vq, monkeypatch):
    """The Python binding checks every tensor it hands to the C ABI: a host
    tensor, a non-contiguous dense buffer, a wrong dtype or a buffer shorter
    than what the call reads or writes raises ValueError before the library
    is called (so no case here reaches a kernel)."""
    import torch
    K, N = 512, 64
    x = torch.zeros(K)
    with pytest.raises(ValueError, match="GPU device memory"):
        vq.gemv(vq.Q4_K, torch.zeros(vq.weight_bytes(vq.Q4_K, N, K), dtype=torch.uint8), N, K, x,
                y=torch.zeros(N))
    with pytest.raises(ValueError, match="GPU device memory"):
        vq.quantize_act(vq.Q8_K, torch.zeros(4, K))
    # The remaining checks hold for any device: let CPU tensors past the
    # device check to reach them (each case still fails before the call).
    monkeypatch.setattr(vq, "_on_gpu", lambda t, name: None)
    W = torch.zeros(vq.weight_bytes(vq.Q4_K, N, K), dtype=torch.uint8)
    with pytest.raises(ValueError, match="W holds"):
        vq.gemv(vq.Q4_K, W[:-1], N, K, x, y=torch.zeros(N))
    with pytest.raises(ValueError, match="x holds"):
        vq.gemv(vq.Q4_K, W, N, K, x[:-4], y=torch.zeros(N))
    with pytest.raises(ValueError, match="x has dtype"):
        vq.gemv(vq.Q4_K, W, N, K, x.double(), y=torch.zeros(N))
    with pytest.raises(ValueError, match="y is not contiguous"):
        vq.gemv(vq.Q4_K, W, N, K, x, y=torch.zeros(N, 2)[:, 0])
    Xq = torch.zeros(vq.act_bytes(vq.Q8_K, 8, K), dtype=torch.uint8)
    with pytest.raises(ValueError, match="Xq holds"):
        vq.gemm(vq.Q4_K, W, N, K, vq.Q8_K, Xq, 9, Y=torch.zeros(9, N))
    with pytest.raises(ValueError, match="do not fit"):
        vq.gemm(vq.Q4_K, W, N, K, vq.Q8_K, Xq, 8, Y=torch.zeros(8 * N)[1:], ldy=N)
    with pytest.raises(ValueError, match="row must be contiguous"):
        vq.quantize_act(vq.Q8_K, torch.zeros(K, 4).t(), M=4, K=K, ldx=1, Xq=Xq)
    with pytest.raises(ValueError, match="do not fit"):
        vq.quantize_act(vq.Q8_K, torch.zeros(4 * K)[K:], M=4, K=K, ldx=K, Xq=Xq)
    T, top_k, E = 4, 2, 8
    ids = torch.zeros(T, top_k, dtype=torch.int64)
    with pytest.raises(ValueError, match="ids has dtype"):
        vq.gemm_grouped(vq.Q4_K, torch.zeros(vq.weight_bytes(vq.Q4_K, E * N, K), dtype=torch.uint8), E, N, K,
                        vq.Q8_K, Xq, T, ids, top_k, route_w=torch.zeros(T, top_k))
    ws = torch.zeros(vq.grouped_workspace_bytes(E, T, top_k) - 256, dtype=torch.uint8)
    with pytest.raises(ValueError, match="ws holds"):
        vq.gemm_grouped(vq.Q4_K, torch.zeros(vq.weight_bytes(vq.Q4_K, E * N, K), dtype=torch.uint8), E, N, K,
                        vq.Q8_K, Xq, T, ids.int(), top_k, route_w=torch.zeros(T, top_k), ws=ws)
    with pytest.raises(ValueError, match="Ysum holds"):
        vq.weighted_sum(torch.zeros(T, top_k, N), torch.zeros(T, top_k), T, top_k, N, Ysum=torch.zeros(T - 1, N))


def test_product_and_oracle_share_no_code():
    """The HIP path and the oracle are independent: no package or kernel
    source names the oracle, the oracle includes or imports nothing of the
    package, and bench.py touches the oracle only in its CPU-baseline leg."""
    pkg = os.path.join(ROOT, "block_quantized_matmul_fp32_amd")
    srcs = [os.path.join(pkg, f) for f in os.listdir(pkg) if f.endswith(".py")]
    srcs += [os.path.join(pkg, "csrc", f) for f in os.listdir(os.path.join(pkg, "csrc"))]
    for path in srcs:
        text = open(path).read()
        assert not re.search(r"^\s*(import oracle|from oracle|#include\s+\S*oracle)", text, flags=re.M), path
    odir = os.path.join(ROOT, "oracle")
    for f in os.listdir(odir):
        if f.endswith((".py", ".c", ".h")):
            text = open(os.path.join(odir, f)).read()
            assert not re.search(r"^\s*(import|from)\s+(block_quantized_matmul_fp32_amd|\.\.)", text, flags=re.M), f
            assert not re.search(r'#include\s+"', text), f  # only system headers
    bench = open(os.path.join(ROOT, "bench.py")).read()
    uses = [m.start() for m in re.finditer(r"\boracle\.|^\s*(import|from) oracle", bench, flags=re.M)]
    assert uses
    for pos in uses:
        func = bench.rfind("\ndef ", 0, pos)
        name = re.match(r"\ndef (\w+)", bench[func:]).group(1) if func >= 0 else "<module>"
        assert "cpu" in name, "bench.py uses the oracle outside its CPU baseline (in %s)" % name


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 exits with status 2 and says so
    (before anything touches a GPU)."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2, r.stderr
    assert "one GPU" in r.stderr and r.stdout == ""
