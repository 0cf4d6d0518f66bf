"""Python binding of the gfx950 attention library (``libfa.so``, C ABI in
``include/fa.h``): forward, first backward and exact backward-over-backward
of softmax attention.

This layer only marshals arguments: it checks tensor shapes and dtypes,
allocates outputs with PyTorch on the inputs' device (the library itself
never allocates), and passes raw device pointers, element strides and the
current HIP stream to the C entry points.  Every step of the computation runs
in the HIP kernels; there is no fallback path.  If the shared library is
missing the calls raise ``FaLibraryError``.
"""
from __future__ import annotations

import ctypes
import os
import warnings

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa.so")

FA_OK = 0
# fa_version() the binding needs: 1.1 added fa_problem.H_kv (an older library
# would read key-side tensors with the query-head count), 1.3 fa_bob_noalloc,
# 1.4 a 64 MiB no-alloc array (NOALLOC_SCRATCH_BYTES below must match).
MIN_VERSION = 10400
STATUS_NAMES = {
    0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_STRIDE", 4: "FA_ERR_DTYPE",
    5: "FA_ERR_UNSUPPORTED", 6: "FA_ERR_WORKSPACE", 7: "FA_ERR_HIP",
}
FA_BF16, FA_FP32 = 0, 1

# Exported symbols (kept equal to the declarations in include/fa.h).
SYMBOLS = ("fa_version", "fa_status_str", "fa_fwd", "fa_bwd_workspace_bytes", "fa_bwd",
           "fa_bob_workspace_bytes", "fa_bob", "fa_bob_noalloc", "fa_bob_phase", "fa_bob_schedule")
# Size of fa_bob_noalloc's static device workspace (FA_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20
# Schedules of fa_bob_schedule (include/fa.h).
SCHED_TWO_PASS, SCHED_TWO_PASS_1WAVE, SCHED_THREE_PASS = 0, 1, 2


class FaLibraryError(RuntimeError):
    pass


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_str(status)})")


class FaProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64),
                ("d", ctypes.c_int64), ("scale", ctypes.c_float), ("causal", ctypes.c_int32),
                ("in_dtype", ctypes.c_int32), ("H_kv", ctypes.c_int64), ("dropout", ctypes.c_float),
                ("reserved", ctypes.c_int32), ("seed", ctypes.c_uint64)]


class FaTensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64)]


_LIB = None


def load_library(path: str | None = None, check_version: bool = True) -> ctypes.CDLL:
    """Load libfa.so (once) and declare the C signatures.  A library older than
    this binding (fa_version() < MIN_VERSION, same major version) is refused."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FaLibraryError(f"{p} is not built; run `python -m exact_second_order_fa_amd.build` "
                             "(hipcc, gfx950) first")
    lib = ctypes.CDLL(p)
    P, T, vp, sz = ctypes.POINTER(FaProblem), FaTensor, ctypes.c_void_p, ctypes.c_size_t
    lib.fa_version.restype = ctypes.c_int
    lib.fa_version.argtypes = []
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_status_str.argtypes = [ctypes.c_int]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_bwd_workspace_bytes.argtypes = [P]
    lib.fa_bob_workspace_bytes.restype = sz
    lib.fa_bob_workspace_bytes.argtypes = [P]
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd.argtypes = [P, T, T, T, T, vp, vp]
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_bwd.argtypes = [P, T, T, T, T, vp, T, T, T, T, vp, sz, vp]
    lib.fa_bob.restype = ctypes.c_int
    lib.fa_bob.argtypes = [P, T, T, T, T, vp, T, T, T, T, T, T, T, T, vp, sz, vp]
    lib.fa_bob_noalloc.restype = ctypes.c_int
    lib.fa_bob_noalloc.argtypes = [P, T, T, T, T, vp, T, T, T, T, T, T, T, T, vp]
    lib.fa_bob_phase.restype = ctypes.c_int
    lib.fa_bob_phase.argtypes = [P, T, T, T, T, vp, T, T, T, T, T, T, T, T, vp, sz, ctypes.c_int32, vp]
    lib.fa_bob_schedule.restype = ctypes.c_int
    lib.fa_bob_schedule.argtypes = [P, T, T, T, T, vp, T, T, T, T, T, T, T, T, vp, sz, ctypes.c_int32,
                                    ctypes.c_int32, vp]
    ver = lib.fa_version()
    if check_version and not (MIN_VERSION <= ver < (MIN_VERSION // 10000 + 1) * 10000):
        raise FaLibraryError(f"{p} has version {ver}; this binding needs {MIN_VERSION} up to the next major "
                             "version (rebuild with `python -m exact_second_order_fa_amd.build`)")
    if path is None:
        _LIB = lib
    return lib


def version() -> int:
    return load_library().fa_version()


def status_str(status: int) -> str:
    return load_library().fa_status_str(int(status)).decode()


# ----------------------------------------------------------------- marshalling

def _torch():
    import torch
    return torch


def problem(B, H, N, d, in_dtype=FA_BF16, scale=None, causal=0, H_kv=0, dropout=0.0, seed=0) -> FaProblem:
    """H: query heads; H_kv: key/value heads (0 = H; otherwise a divisor of H);
    dropout: rate p in [0, 1) with generator key ``seed`` (the same pair for
    fa_fwd, fa_bwd and fa_bob).  The library keeps an element with
    probability 1 - t/256, t = round(256 p): p is used as the nearest
    multiple of 1/256 (p = 0.1 drops 26/256), and 0 < p < 1/512 rounds to
    t = 0, i.e. no dropout (a warning says so)."""
    p = float(dropout)
    if 0.0 < p < 0.5 / 256:
        warnings.warn(f"dropout rate {p} rounds to threshold 0 of 256: no element is dropped", stacklevel=3)
    return FaProblem(int(B), int(H), int(N), int(d), float(-1.0 if scale is None else scale),
                     int(causal), int(in_dtype), int(H_kv), p, 0, int(seed) & (2 ** 64 - 1))


def tensor_arg(t) -> FaTensor:
    """An fa_tensor for a [B, H, N, d] torch tensor with a contiguous last dim."""
    if t.dim() != 4:
        raise ValueError(f"expected a [B, H, N, d] tensor, got shape {tuple(t.shape)}")
    if t.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous (stride 1)")
    return FaTensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_FP32
    raise TypeError(f"inputs must be bfloat16 or float32, got {t.dtype}")


def _check_inputs(qside, kside):
    """Query-side tensors [B, H, N, d] and key-side tensors [B, H_kv, N, d]
    (H_kv dividing H) of one dtype on one device; returns (B, H, N, d, H_kv)."""
    q0, k0 = qside[0], kside[0]
    for group, ref in ((qside, q0), (kside, k0)):
        for t in group:
            if t.shape != ref.shape or t.dtype != q0.dtype or t.device != q0.device:
                raise ValueError("q, dout and U_Q (and k, v, U_K, U_V) must share shape; all inputs share "
                                 "dtype and device")
            if not t.is_cuda:
                raise ValueError("tensors must live on the GPU")
    B, H, N, d = q0.shape
    Bk, Hkv, Nk, dk = k0.shape
    if (Bk, Nk, dk) != (B, N, d) or Hkv < 1 or H % Hkv:
        raise ValueError(f"key-side shape {tuple(k0.shape)} does not match query-side shape {tuple(q0.shape)} "
                         "(same B, N, d; key/value heads must divide query heads)")
    return B, H, N, d, Hkv


def _stream(stream):
    torch = _torch()
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _keep_for_stream(stream, allocated):
    """Tensors this binding allocated on torch's current stream but handed to
    kernels on another stream: record that stream on them, so the caching
    allocator does not reuse their memory before those kernels finish."""
    torch = _torch()
    if stream is None:
        return
    if isinstance(stream, int):
        if stream == torch.cuda.current_stream().cuda_stream:
            return
        stream = torch.cuda.ExternalStream(stream)
    elif stream.cuda_stream == torch.cuda.current_stream().cuda_stream:
        return
    for t in allocated:
        t.record_stream(stream)


def _f32_like(x, out, what):
    """A float32 tensor shaped like x on x's device: ``out`` after checking
    it, or a new one (second return value: whether it was allocated here)."""
    torch = _torch()
    if out is not None:
        if out.dtype != torch.float32 or out.shape != x.shape or out.device != x.device:
            raise ValueError(f"{what} must be float32 with shape {tuple(x.shape)} on {x.device}")
        return out, False
    return torch.empty(x.shape, dtype=torch.float32, device=x.device), True


def _check_saved_state(q, o, lse):
    """O from fa_fwd: float32, q's shape and device; L: a contiguous float32
    [B, H, N] tensor on q's device (the library reads it by raw pointer)."""
    torch = _torch()
    B, H, N, _ = q.shape
    if o.dtype != torch.float32 or o.shape != q.shape or o.device != q.device:
        raise ValueError(f"o must be the float32 forward output with shape {tuple(q.shape)} on {q.device}")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or lse.device != q.device \
            or not lse.is_contiguous():
        raise ValueError(f"lse must be a contiguous float32 tensor of shape {(B, H, N)} on {q.device}")


def _call(name, status):
    if status != FA_OK:
        raise FaError(status, name)


def fa_fwd(q, k, v, scale=None, o=None, lse=None, stream=None, causal=False, dropout=0.0, seed=0):
    """Forward: returns (O fp32 [B,H,N,d], L fp32 [B,H,N], natural-log
    log-sum-exp of tau q.k over the (causally) valid keys).  k, v may have
    fewer heads than q (grouped-query / multi-query attention).  With
    ``dropout`` > 0, O = (P * g) V for the keep mask g of (dropout, seed);
    the rate is rounded to a multiple of 1/256 (see ``problem``)."""
    torch = _torch()
    B, H, N, d, Hkv = _check_inputs((q,), (k, v))
    p = problem(B, H, N, d, _dtype_code(q), scale, int(bool(causal)), Hkv, dropout, seed)
    o, new_o = _f32_like(q, o, "o")
    allocated = [o] if new_o else []
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        allocated.append(lse)
    else:
        _check_saved_state(q, o, lse)
    lib = load_library()
    _keep_for_stream(stream, allocated)
    _call("fa_fwd", lib.fa_fwd(ctypes.byref(p), tensor_arg(q), tensor_arg(k), tensor_arg(v),
                               tensor_arg(o), ctypes.c_void_p(lse.data_ptr()), _stream(stream)))
    return o, lse


def bwd_workspace_bytes(B, H, N, d, in_dtype=FA_BF16, causal=False, H_kv=0) -> int:
    p = problem(B, H, N, d, in_dtype, None, int(bool(causal)), H_kv)
    return int(load_library().fa_bwd_workspace_bytes(ctypes.byref(p)))


def bob_workspace_bytes(B, H, N, d, in_dtype=FA_BF16, causal=False, H_kv=0) -> int:
    """Bytes of fa_bob's workspace (it depends on H_kv: grouped-query
    problems with few key blocks also hold the column pass's partial sums)."""
    p = problem(B, H, N, d, in_dtype, None, int(bool(causal)), H_kv)
    return int(load_library().fa_bob_workspace_bytes(ctypes.byref(p)))


def _workspace(nbytes, device, ws):
    """A caller's workspace after checking it, or a new one (second return
    value: whether it was allocated here)."""
    torch = _torch()
    if ws is None:
        return torch.empty(max(nbytes, 16) // 4, dtype=torch.float32, device=device), True
    if ws.device != device or not ws.is_contiguous():
        raise ValueError(f"the workspace must be a contiguous tensor on {device}")
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace too small: {ws.numel() * ws.element_size()} < {nbytes} bytes")
    return ws, False


def fa_bwd(q, k, v, o, lse, dout, scale=None, dq=None, dk=None, dv=None, ws=None, stream=None,
           causal=False, dropout=0.0, seed=0):
    """First backward: returns (dQ, dK, dV) fp32 and the workspace holding D.
    dK, dV have k's heads (sums over each group's query heads).  ``dropout``
    and ``seed`` must be the forward's."""
    B, H, N, d, Hkv = _check_inputs((q, dout), (k, v))
    _check_saved_state(q, o, lse)
    p = problem(B, H, N, d, _dtype_code(q), scale, int(bool(causal)), Hkv, dropout, seed)
    outs = [_f32_like(q, dq, "dq"), _f32_like(k, dk, "dk"), _f32_like(k, dv, "dv")]
    dq, dk, dv = (t for t, _ in outs)
    nbytes = int(load_library().fa_bwd_workspace_bytes(ctypes.byref(p)))
    ws, new_ws = _workspace(nbytes, q.device, ws)
    _keep_for_stream(stream, [t for t, new in outs + [(ws, new_ws)] if new])
    _call("fa_bwd", load_library().fa_bwd(
        ctypes.byref(p), tensor_arg(q), tensor_arg(k), tensor_arg(v), tensor_arg(o),
        ctypes.c_void_p(lse.data_ptr()), tensor_arg(dout), tensor_arg(dq), tensor_arg(dk),
        tensor_arg(dv), ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel() * ws.element_size()),
        _stream(stream)))
    return dq, dk, dv, ws


def fa_bob(q, k, v, o, lse, dout, uq, uk, uv, scale=None, gq=None, gk=None, gv=None, gdo=None,
           ws=None, stream=None, phase=None, causal=False, schedule=None, dropout=0.0, seed=0):
    """Backward-over-backward: gradients of <dQ,U_Q> + <dK,U_K> + <dV,U_V> with
    respect to Q, K, V and dO (k, v, uk, uv and gK, gV may have fewer heads
    than q: grouped-query / multi-query attention).  Returns (gQ, gK, gV, gdO, ws) with
    ws = [D | alpha | E], each [B, H, N] fp32.  ``phase`` (0, 1 or 2) calls
    fa_bob_phase instead, launching only that kernel.  ``schedule`` (one of
    the SCHED_* constants) calls fa_bob_schedule: the schedule ablation of
    the pages' appendix G.1 (phases 0-3 for the three-pass schedule).
    ``dropout`` and ``seed`` must be the forward's (the pages' analytical
    dropout extension)."""
    B, H, N, d, Hkv = _check_inputs((q, dout, uq), (k, v, uk, uv))
    _check_saved_state(q, o, lse)
    p = problem(B, H, N, d, _dtype_code(q), scale, int(bool(causal)), Hkv, dropout, seed)
    outs = [_f32_like(q, gq, "gq"), _f32_like(k, gk, "gk"), _f32_like(k, gv, "gv"), _f32_like(q, gdo, "gdo")]
    gq, gk, gv, gdo = (t for t, _ in outs)
    lib = load_library()
    nbytes = int(lib.fa_bob_workspace_bytes(ctypes.byref(p)))
    ws, new_ws = _workspace(nbytes, q.device, ws)
    _keep_for_stream(stream, [t for t, new in outs + [(ws, new_ws)] if new])
    args = [ctypes.byref(p), tensor_arg(q), tensor_arg(k), tensor_arg(v), tensor_arg(o),
            ctypes.c_void_p(lse.data_ptr()), tensor_arg(dout), tensor_arg(uq), tensor_arg(uk),
            tensor_arg(uv), tensor_arg(gq), tensor_arg(gk), tensor_arg(gv), tensor_arg(gdo),
            ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel() * ws.element_size())]
    if schedule is not None:
        _call("fa_bob_schedule", lib.fa_bob_schedule(*args, ctypes.c_int32(schedule),
                                                      ctypes.c_int32(-1 if phase is None else phase),
                                                      _stream(stream)))
    elif phase is None:
        _call("fa_bob", lib.fa_bob(*args, _stream(stream)))
    else:
        _call("fa_bob_phase", lib.fa_bob_phase(*args, ctypes.c_int32(phase), _stream(stream)))
    return gq, gk, gv, gdo, ws


def fa_bob_noalloc(q, k, v, o, lse, dout, uq, uk, uv, gq, gk, gv, gdo, scale=None, stream=None, causal=False,
                   dropout=0.0, seed=0):
    """fa_bob without a workspace, for callers that must not allocate device
    memory: the library keeps D, alpha, E in a static device array of
    NOALLOC_SCRATCH_BYTES per GPU (so they are not returned), and this
    function allocates nothing either, so every output (gq, gdo with q's
    shape; gk, gv with k's) must be given.  Calls that overlap on one GPU
    share that array and must be serialised.  Returns (gq, gk, gv, gdo)."""
    B, H, N, d, Hkv = _check_inputs((q, dout, uq), (k, v, uk, uv))
    _check_saved_state(q, o, lse)
    if any(t is None for t in (gq, gk, gv, gdo)):
        raise ValueError("fa_bob_noalloc allocates nothing: pass gq, gk, gv and gdo")
    for t, like, what in ((gq, q, "gq"), (gk, k, "gk"), (gv, k, "gv"), (gdo, q, "gdo")):
        _f32_like(like, t, what)
    p = problem(B, H, N, d, _dtype_code(q), scale, int(bool(causal)), Hkv, dropout, seed)
    _call("fa_bob_noalloc", load_library().fa_bob_noalloc(
        ctypes.byref(p), tensor_arg(q), tensor_arg(k), tensor_arg(v), tensor_arg(o),
        ctypes.c_void_p(lse.data_ptr()), tensor_arg(dout), tensor_arg(uq), tensor_arg(uk), tensor_arg(uv),
        tensor_arg(gq), tensor_arg(gk), tensor_arg(gv), tensor_arg(gdo), _stream(stream)))
    return gq, gk, gv, gdo


def split_workspace(ws, B, H, N):
    """Views D, alpha, E of a fa_bob workspace."""
    n = B * H * N
    return ws[:n].view(B, H, N), ws[n:2 * n].view(B, H, N), ws[2 * n:3 * n].view(B, H, N)
