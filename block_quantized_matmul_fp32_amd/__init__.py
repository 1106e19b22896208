"""Python binding of the gfx950 block-quantized matmul library (include/vq.h).

Argument marshalling only: every function passes device pointers, sizes and
the current HIP stream to the C ABI of ``libvq.so`` and raises ``VQError``
on a non-OK status.  PyTorch supplies device memory and streams; no step of
the computation runs in Python or on the CPU.  If the library is not built
(``python -m block_quantized_matmul_fp32_amd.build``) every call fails loudly.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libvq.so")

Q4_K, Q6_K, Q8_0, Q8_K, Q8_1, Q5_K = 0, 1, 2, 3, 4, 5
TYPE_NAMES = {Q4_K: "Q4_K", Q6_K: "Q6_K", Q8_0: "Q8_0", Q8_K: "Q8_K", Q8_1: "Q8_1"}
OP_GEMV, OP_GEMM, OP_GEMM_GROUPED = 0, 1, 2

STATUS = {0: "VQ_OK", 1: "VQ_ERR_INVALID_ARG", 2: "VQ_ERR_UNSUPPORTED_TYPE", 3: "VQ_ERR_TYPE_PAIR",
          4: "VQ_ERR_SHAPE", 5: "VQ_ERR_ALIAS", 6: "VQ_ERR_WORKSPACE", 7: "VQ_ERR_HIP", 8: "VQ_ERR_DEVICE"}
DEBUG_SYNC = 1
DEBUG_CHECK_IDS = 2

EXPORTS = [
    "vq_status_string", "vq_last_error", "vq_type_name", "vq_is_supported", "vq_block_values",
    "vq_block_bytes", "vq_weight_bytes", "vq_act_bytes", "vq_act_d_offset", "vq_act_aux_offset",
    "vq_quantize_act", "vq_quantize_weights", "vq_gemv", "vq_gemm", "vq_grouped_workspace_bytes",
    "vq_gemm_grouped", "vq_gemm_grouped_rows", "vq_gemm_grouped_noalloc", "vq_stream_probe", "vq_weighted_sum", "vq_get_stats", "vq_reset_stats",
    "vq_version", "vq_rmsnorm_quant", "vq_silu_mul_quant", "vq_set_small_batch_max", "vq_small_batch_max",
    "vq_set_gemm_row_block", "vq_gemm_workspace", "vq_set_debug", "vq_device_status", "vq_mfma_probe",
]

STAT_FIELDS = ["quantize_q8k", "quantize_q8_1", "quantize_weights", "gemv_q4k", "gemv_q6k", "gemv_q8_0",
               "gemm_q4k", "gemm_q6k", "gemm_q8_0", "route", "gemm_grouped_q4k", "weighted_sum",
               "gemm_grouped_q6k", "gemm_grouped_q8_0", "gemm_grouped_rows", "gemm_skinny",
               "gemv_q5k", "gemm_q5k", "gemm_grouped_q5k", "rmsnorm_quant", "silu_mul_quant"]


class VQStats(ctypes.Structure):
    _fields_ = [(f, ctypes.c_uint64) for f in STAT_FIELDS]


class VQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS.get(status, str(status)), message))
        self.status = status
        self.status_name = STATUS.get(status, str(status))
        self.message = message


_lib = None


def lib():
    """The loaded libvq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libvq.so is not built (python -m block_quantized_matmul_fp32_amd.build); "
                              "there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I, Z = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        L.vq_status_string.restype = ctypes.c_char_p
        L.vq_status_string.argtypes = [I]
        L.vq_last_error.restype = ctypes.c_char_p
        L.vq_type_name.restype = ctypes.c_char_p
        L.vq_type_name.argtypes = [I]
        L.vq_is_supported.argtypes = [I, I, I]
        L.vq_block_values.argtypes = [I]
        L.vq_block_bytes.argtypes = [I]
        L.vq_block_bytes.restype = Z
        for f in ("vq_weight_bytes", "vq_act_bytes", "vq_act_d_offset", "vq_act_aux_offset"):
            getattr(L, f).argtypes = [I, I64, I64]
            getattr(L, f).restype = Z
        L.vq_quantize_act.argtypes = [I, P, I64, I64, I64, P, P]
        L.vq_quantize_weights.argtypes = [I, P, I64, I64, P, P]
        L.vq_gemv.argtypes = [I, P, I64, I64, P, P, P, P]
        L.vq_gemm.argtypes = [I, P, I64, I64, I, P, I64, P, I64, P, Z, P]
        L.vq_gemm_workspace.argtypes = [I, I64, I64, I64]
        L.vq_gemm_workspace.restype = Z
        L.vq_grouped_workspace_bytes.argtypes = [I64, I64, I64]
        L.vq_grouped_workspace_bytes.restype = Z
        L.vq_gemm_grouped.argtypes = [I, P, I64, I64, I64, I, P, I64, P, I64, P, P, P, P, Z, P]
        L.vq_gemm_grouped_rows.argtypes = [I, P, I64, I64, I64, I, P, I64, P, I64, P, P, P, P, Z, P]
        L.vq_gemm_grouped_noalloc.argtypes = [I, P, I64, I64, I64, I, P, I64, P, I64, P, P, P, P]
        L.vq_stream_probe.argtypes = [I, P, I64, I64, P, Z, P]
        L.vq_mfma_probe.argtypes = [I64, P, Z, ctypes.POINTER(ctypes.c_int64), P]
        L.vq_mfma_probe.restype = I
        L.vq_set_debug.argtypes = [I, I64]
        L.vq_set_debug.restype = I
        L.vq_device_status.argtypes = [P]
        L.vq_device_status.restype = I
        L.vq_weighted_sum.argtypes = [P, P, I64, I64, I64, P, P]
        L.vq_set_small_batch_max.argtypes = [I, I64]
        L.vq_set_small_batch_max.restype = I
        L.vq_small_batch_max.argtypes = [I]
        L.vq_small_batch_max.restype = I64
        L.vq_set_gemm_row_block.argtypes = [I64]
        L.vq_set_gemm_row_block.restype = I
        L.vq_rmsnorm_quant.argtypes = [I, P, P, I64, I64, I64, ctypes.c_float, P, I64, P, P]
        L.vq_silu_mul_quant.argtypes = [I, P, P, I64, I64, I64, P, I64, P, P]
        L.vq_get_stats.argtypes = [ctypes.POINTER(VQStats)]
        L.vq_version.restype = ctypes.c_char_p
        for f in ("vq_quantize_act", "vq_quantize_weights", "vq_gemv", "vq_gemm", "vq_gemm_grouped",
                  "vq_gemm_grouped_rows", "vq_gemm_grouped_noalloc", "vq_stream_probe", "vq_weighted_sum", "vq_rmsnorm_quant", "vq_silu_mul_quant"):
            getattr(L, f).restype = I
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise VQError(status, lib().vq_last_error().decode())


def _on_gpu(t, name):
    if t.device.type != "cuda":
        raise ValueError("%s is on %s: the library takes GPU device memory" % (name, t.device))


def _dev(t, name, nbytes=None, dtype=None):
    """Device address of a dense buffer argument.  A tensor must be on a GPU,
    contiguous, of the given dtype and at least nbytes long, so that the
    kernels never touch memory outside it; None and raw integer addresses
    pass through unchecked."""
    if t is None or isinstance(t, int):
        return t
    _on_gpu(t, name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s has dtype %s, %s expected" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s is not contiguous" % name)
    if nbytes is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError("%s holds %d bytes, %d needed" % (name, t.numel() * t.element_size(), nbytes))
    return t.data_ptr()


def _dev_rows(t, name, M, K, ld, dtype=None):
    """Device address of a row-strided fp32 argument (rows of K values, ld
    apart): on a GPU, unit stride inside a row, and (M - 1) * ld + K values
    inside the tensor's storage."""
    if t is None or isinstance(t, int):
        return t
    _on_gpu(t, name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s has dtype %s, %s expected" % (name, t.dtype, dtype))
    if t.dim() >= 1 and t.numel() > 1 and t.stride(-1) != 1:
        raise ValueError("%s: the values of a row must be contiguous" % name)
    avail = t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()
    if M > 0 and (M - 1) * ld + K > avail:
        raise ValueError("%s: %d rows of %d values, %d apart, do not fit its storage" % (name, M, K, ld))
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _torch():
    import torch
    return torch


# ------------------------------------------------------------------- sizes
def block_values(t: int) -> int:
    return lib().vq_block_values(t)


def block_bytes(t: int) -> int:
    return lib().vq_block_bytes(t)


def weight_bytes(w: int, N: int, K: int) -> int:
    return lib().vq_weight_bytes(w, N, K)


def act_bytes(act: int, M: int, K: int) -> int:
    return lib().vq_act_bytes(act, M, K)


def act_d_offset(act: int, M: int, K: int) -> int:
    return lib().vq_act_d_offset(act, M, K)


def act_aux_offset(act: int, M: int, K: int) -> int:
    return lib().vq_act_aux_offset(act, M, K)


def set_small_batch_max(w: int, max_m: int):
    """vq_set_small_batch_max: vq_gemm runs M <= max_m on the GEMV kernel (-1: default)."""
    _check(lib().vq_set_small_batch_max(w, max_m))


def small_batch_max(w: int) -> int:
    return int(lib().vq_small_batch_max(w))


def set_gemm_row_block(rows: int):
    """vq_set_gemm_row_block: cap the rows of one MFMA GEMM launch (0: default)."""
    _check(lib().vq_set_gemm_row_block(rows))


def grouped_workspace_bytes(E: int, T: int, top_k: int) -> int:
    return lib().vq_grouped_workspace_bytes(E, T, top_k)


def is_supported(w: int, act: int, op: int) -> bool:
    return bool(lib().vq_is_supported(w, act, op))


def type_name(t: int) -> str:
    return lib().vq_type_name(t).decode()


def version() -> str:
    return lib().vq_version().decode()


def act_for(w: int) -> int:
    """The activation type a weight type pairs with."""
    return Q8_1 if w == Q8_0 else Q8_K


# ------------------------------------------------------------------- calls
def quantize_act(act: int, X, M: int = None, K: int = None, ldx: int = None, Xq=None, stream=None):
    """vq_quantize_act: fp32 X [M, ldx] -> planar Q8_K / Q8_1 bytes (uint8 tensor)."""
    if M is None:
        M, K = (1, X.shape[0]) if X.dim() == 1 else (X.shape[0], X.shape[1])
    if ldx is None:
        ldx = K if X.dim() == 1 or X.shape[0] == 1 else X.stride(0)
    if Xq is None:
        Xq = _torch().empty(act_bytes(act, M, K), dtype=_torch().uint8, device=X.device)
    f32, u8 = _torch().float32, _torch().uint8
    _check(lib().vq_quantize_act(act, _dev_rows(X, "X", M, K, ldx, f32), M, K, ldx,
                                 _dev(Xq, "Xq", act_bytes(act, M, K), u8), _stream(stream)))
    return Xq


def _rows(X, M, K, ldx):
    if M is None:
        M, K = (1, X.shape[0]) if X.dim() == 1 else (X.shape[0], X.shape[1])
    if ldx is None:
        # a single row may carry any stride in its leading dimension
        ldx = K if X.dim() == 1 or X.shape[0] == 1 else X.stride(0)
    return M, K, ldx


def rmsnorm_quant(act: int, X, gamma, eps: float = 1e-6, M: int = None, K: int = None, ldx: int = None,
                  Y=None, want_y: bool = True, ldy: int = None, Xq=None, stream=None):
    """vq_rmsnorm_quant: (Y, Xq) with Y = RMSNorm(X) * gamma (None if not
    wanted) and Xq its planar Q8_K / Q8_1 bytes, from one launch."""
    M, K, ldx = _rows(X, M, K, ldx)
    torch = _torch()
    if Y is None and want_y:
        Y = torch.empty((M, K), dtype=torch.float32, device=X.device)
    if ldy is None:
        ldy = K if Y is None or Y.dim() == 1 or Y.shape[0] == 1 else Y.stride(0)
    if Xq is None:
        Xq = torch.empty(act_bytes(act, M, K), dtype=torch.uint8, device=X.device)
    f32 = torch.float32
    _check(lib().vq_rmsnorm_quant(act, _dev_rows(X, "X", M, K, ldx, f32), _dev(gamma, "gamma", 4 * K, f32), M, K,
                                  ldx, float(eps), _dev_rows(Y, "Y", M, K, ldy, f32), ldy,
                                  _dev(Xq, "Xq", act_bytes(act, M, K), torch.uint8), _stream(stream)))
    return Y, Xq


def silu_mul_quant(act: int, G, U, M: int = None, K: int = None, ldx: int = None, Y=None, want_y: bool = True,
                   ldy: int = None, Xq=None, stream=None):
    """vq_silu_mul_quant: (Y, Xq) with Y = silu(G) * U (None if not wanted)
    and Xq its planar Q8_K / Q8_1 bytes, from one launch."""
    M, K, ldx = _rows(G, M, K, ldx)
    torch = _torch()
    if Y is None and want_y:
        Y = torch.empty((M, K), dtype=torch.float32, device=G.device)
    if ldy is None:
        ldy = K if Y is None or Y.dim() == 1 or Y.shape[0] == 1 else Y.stride(0)
    if Xq is None:
        Xq = torch.empty(act_bytes(act, M, K), dtype=torch.uint8, device=G.device)
    f32 = torch.float32
    _check(lib().vq_silu_mul_quant(act, _dev_rows(G, "G", M, K, ldx, f32), _dev_rows(U, "U", M, K, ldx, f32), M, K,
                                   ldx, _dev_rows(Y, "Y", M, K, ldy, f32), ldy,
                                   _dev(Xq, "Xq", act_bytes(act, M, K), torch.uint8), _stream(stream)))
    return Y, Xq


def quantize_weights(w: int, W, N: int = None, K: int = None, Wq=None, stream=None):
    """vq_quantize_weights: fp32 W [N, K] -> block bytes (uint8 tensor)."""
    if N is None:
        N, K = W.shape
    if Wq is None:
        Wq = _torch().empty(weight_bytes(w, N, K), dtype=_torch().uint8, device=W.device)
    _check(lib().vq_quantize_weights(w, _dev(W, "W", 4 * N * K, _torch().float32), N, K,
                                     _dev(Wq, "Wq", weight_bytes(w, N, K)), _stream(stream)))
    return Wq


def gemv(w: int, W, N: int, K: int, x, y=None, xq_out=None, stream=None):
    """vq_gemv: y[N] = W . x with the activation quantizer fused in."""
    if y is None:
        y = _torch().empty(N, dtype=_torch().float32, device=x.device)
    f32 = _torch().float32
    _check(lib().vq_gemv(w, _dev(W, "W", weight_bytes(w, N, K)), N, K, _dev(x, "x", 4 * K, f32),
                         _dev(y, "y", 4 * N, f32), _dev(xq_out, "xq_out", act_bytes(act_for(w), 1, K)),
                         _stream(stream)))
    return y


def gemm_workspace(w: int, M: int, N: int, K: int) -> int:
    """vq_gemm_workspace: bytes of split-K workspace vq_gemm wants for this shape."""
    return int(lib().vq_gemm_workspace(w, M, N, K))


_ws_cache = {}


def _gemm_ws(dev, stream_handle, nbytes):
    """A zero-filled workspace of at least nbytes, kept per (device, stream):
    vq_gemm leaves its counters zero after each call, so calls on one stream
    can reuse it (they run in order)."""
    if nbytes == 0:
        return None
    key = (str(dev), stream_handle)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        torch = _torch()
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _ws_cache[key] = ws
    return ws


def gemm(w: int, W, N: int, K: int, act: int, Xq, M: int, Y=None, ldy: int = None, ws="auto", stream=None):
    """vq_gemm: Y[M, N] = deq(Xq) . deq(W)^T.  ws: "auto" (a zero-filled
    workspace kept per device and stream), None (no split K), or a uint8
    device tensor (zero-filled before its first use)."""
    if Y is None:
        Y = _torch().empty((M, N), dtype=_torch().float32, device=Xq.device)
    if ldy is None:
        ldy = N if Y.dim() == 1 or Y.shape[0] == 1 else Y.stride(0)
    pw = _dev(W, "W", weight_bytes(w, N, K))
    px = _dev(Xq, "Xq", act_bytes(act, M, K))
    py = _dev_rows(Y, "Y", M, N, ldy, _torch().float32)
    sh = _stream(stream)
    if isinstance(ws, str):
        ws = _gemm_ws(Xq.device, sh, gemm_workspace(w, M, N, K))
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().vq_gemm(w, pw, N, K, act, px, M, py, ldy, _dev(ws, "ws", wsb, _torch().uint8), wsb, sh))
    return Y


def gemm_grouped(w: int, W, E: int, N: int, K: int, act: int, Xq, T: int, ids, top_k: int,
                 route_w=None, Y=None, Ysum=None, ws=None, want_sum: bool = True, stream=None,
                 per_row: bool = False):
    """vq_gemm_grouped (or, with per_row, vq_gemm_grouped_rows: Xq holds one
    row per (t, s) pair): Y[T, top_k, N] and (optionally) Ysum[T, N]; returns
    (Y, Ysum, ws)."""
    torch = _torch()
    dev = Xq.device
    if Y is None:
        Y = torch.empty((T, top_k, N), dtype=torch.float32, device=dev)
    if Ysum is None and want_sum and route_w is not None:
        Ysum = torch.empty((T, N), dtype=torch.float32, device=dev)
    need = grouped_workspace_bytes(E, T, top_k)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    fn = lib().vq_gemm_grouped_rows if per_row else lib().vq_gemm_grouped
    f32 = torch.float32
    pairs = T * top_k
    _check(fn(w, _dev(W, "W", weight_bytes(w, E * N, K)), E, N, K, act,
              _dev(Xq, "Xq", act_bytes(act, pairs if per_row else T, K)), T, _dev(ids, "ids", 4 * pairs, torch.int32),
              top_k, _dev(route_w, "route_w", 4 * pairs, f32), _dev(Y, "Y", 4 * pairs * N, f32),
              _dev(Ysum, "Ysum", 4 * T * N, f32), _dev(ws, "ws", need), ws.numel() * ws.element_size() if hasattr(ws, "numel") else need,
              _stream(stream)))
    return Y, Ysum, ws


def set_debug(flags: int = 0, wait_polls: int = 0):
    """vq_set_debug for the calling thread (DEBUG_SYNC, DEBUG_CHECK_IDS)."""
    _check(lib().vq_set_debug(flags, wait_polls))


def device_status(stream=None):
    """vq_device_status: raises VQError(VQ_ERR_DEVICE) if a kernel reported a
    failure since the last check (and clears the report)."""
    _check(lib().vq_device_status(_stream(stream)))


def stream_probe(w: int, W, N: int, K: int, sink, stream=None):
    """vq_stream_probe: read the decode GEMV's weight bytes with its launch
    shape and nothing else (the streaming floor of that launch)."""
    nb = sink.numel() * sink.element_size()
    _check(lib().vq_stream_probe(w, _dev(W, "W", weight_bytes(w, N, K)), N, K, _dev(sink, "sink", 4 * N), nb,
                                 _stream(stream)))


def mfma_probe(iters: int, sink, stream=None) -> int:
    """vq_mfma_probe: the int8 MFMA ceiling launch (register operands, eight
    chains per wave, nothing else); returns the int8 operations it performs."""
    addr = _dev(sink, "sink", 4)
    ops = ctypes.c_int64(0)
    _check(lib().vq_mfma_probe(int(iters), addr, sink.numel() * sink.element_size(), ctypes.byref(ops),
                               _stream(stream)))
    return ops.value


GROUPED_NOALLOC_SCRATCH_BYTES = 4 << 20  # VQ_GROUPED_NOALLOC_SCRATCH_BYTES


def gemm_grouped_noalloc(w: int, W, E: int, N: int, K: int, act: int, Xq, T: int, ids, top_k: int,
                         route_w, Y, Ysum=None, stream=None):
    """vq_gemm_grouped_noalloc: the broadcast arm with its routing workspace in
    the library's static per-GPU scratch array.  Y (and Ysum, if wanted) are
    the caller's: this wrapper allocates nothing either."""
    torch = _torch()
    f32 = torch.float32
    pairs = T * top_k
    _check(lib().vq_gemm_grouped_noalloc(
        w, _dev(W, "W", weight_bytes(w, E * N, K)), E, N, K, act, _dev(Xq, "Xq", act_bytes(act, T, K)), T,
        _dev(ids, "ids", 4 * pairs, torch.int32), top_k, _dev(route_w, "route_w", 4 * pairs, f32),
        _dev(Y, "Y", 4 * pairs * N, f32), _dev(Ysum, "Ysum", 4 * T * N, f32), _stream(stream)))
    return Y, Ysum


def weighted_sum(Y, route_w, T: int, top_k: int, N: int, Ysum=None, stream=None):
    """vq_weighted_sum: Ysum[T, N] = sum_s w[t, s] * Y[t, s, :] (slot order, no FMA)."""
    if Ysum is None:
        Ysum = _torch().empty((T, N), dtype=_torch().float32, device=Y.device)
    f32 = _torch().float32
    _check(lib().vq_weighted_sum(_dev(Y, "Y", 4 * T * top_k * N, f32), _dev(route_w, "route_w", 4 * T * top_k, f32),
                                 T, top_k, N, _dev(Ysum, "Ysum", 4 * T * N, f32), _stream(stream)))
    return Ysum


def get_stats() -> dict:
    s = VQStats()
    lib().vq_get_stats(ctypes.byref(s))
    return {f: int(getattr(s, f)) for f in STAT_FIELDS}


def reset_stats():
    lib().vq_reset_stats()


def grouped_ws_views(ws, E: int, T: int, top_k: int):
    """counts [E], offsets [E+1], list [T*top_k] views into a workspace after a
    vq_gemm_grouped call (section layout of include/vq.h)."""
    torch = _torch()

    def a256(x):
        return (x + 255) // 256 * 256

    o_counts = 0
    o_offsets = a256(4 * E)
    o_list = o_offsets + a256(4 * (E + 1))
    w32 = ws.view(torch.int32)
    return (w32[o_counts // 4:o_counts // 4 + E], w32[o_offsets // 4:o_offsets // 4 + E + 1],
            w32[o_list // 4:o_list // 4 + T * top_k])
