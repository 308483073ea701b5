"""Python binding of libgdn.so (the C ABI in include/gdn.h).

Argument marshalling only: every step of the recurrence runs in the library's
HIP kernels.  PyTorch provides device memory and the current HIP stream; the
functions here check dtypes, shapes and contiguity, allocate outputs and the
workspace with torch when the caller does not pass them, and hand raw
pointers to the library.  There is no fallback: if libgdn.so is missing or
fails to load, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# GDN_LIB_PATH selects another build of the same library (e.g. one whose host
# code carries sanitizers); by default the in-tree libgdn.so.
LIB_PATH = os.environ.get("GDN_LIB_PATH") or os.path.join(_HERE, "libgdn.so")

GDN_F32 = 0
GDN_BF16 = 1
CHUNK = 64
HEAD_DIM = 128

_STATUS = {0: "GDN_OK", -1: "GDN_ERR_NULL", -2: "GDN_ERR_SHAPE", -3: "GDN_ERR_UNSUPPORTED",
           -4: "GDN_ERR_ALIGN", -5: "GDN_ERR_ALIAS", -6: "GDN_ERR_WORKSPACE", -7: "GDN_ERR_HIP"}


class GDNError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libgdn.so not found at %s; build it with "
            "`python -m hybrid_linear_attention_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_float
    pre = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int, vp, sz, vp]
    for name in ("gdn_prefill_chunked", "gdn_prefill_prepare", "gdn_prefill_scan",
                 "gdn_prefill_chunked_bf16_state"):
        fn = getattr(lib, name)
        fn.argtypes = pre
        fn.restype = ctypes.c_int
    lib.gdn_prefill_chunked_noalloc.argtypes = pre[:14] + [vp]
    lib.gdn_prefill_chunked_noalloc.restype = ctypes.c_int
    lib.gdn_prefill_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int]
    lib.gdn_prefill_workspace_bytes.restype = sz
    lib.gdn_varlen_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int]
    lib.gdn_varlen_workspace_bytes.restype = sz
    lib.gdn_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                    ctypes.c_int, vp]
    lib.gdn_decode_step.restype = ctypes.c_int
    lib.gdn_decode_step_bf16_state.argtypes = lib.gdn_decode_step.argtypes
    lib.gdn_decode_step_bf16_state.restype = ctypes.c_int
    lib.gdn_decode_verify.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                      ctypes.c_int, vp]
    lib.gdn_decode_verify.restype = ctypes.c_int
    lib.gdn_decode_commit.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                      ctypes.c_int, vp]
    lib.gdn_decode_commit.restype = ctypes.c_int
    lib.gdn_prefill_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp,
                                       f32, i32, i32, i32, ctypes.c_int, vp, sz, vp]
    lib.gdn_prefill_varlen.restype = ctypes.c_int
    lib.gdn_prefill_chunked_bwd.argtypes = [vp] * 14 + [i32] * 5 + [ctypes.c_int, vp, sz, vp]
    lib.gdn_prefill_chunked_bwd.restype = ctypes.c_int
    lib.gdn_prefill_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int]
    lib.gdn_prefill_bwd_workspace_bytes.restype = sz
    lib.gdn_prefill_varlen_bwd.argtypes = ([vp] * 6 + [i32, i32] + [vp] * 9 + [i32] * 3
                                           + [ctypes.c_int, vp, sz, vp])
    lib.gdn_prefill_varlen_bwd.restype = ctypes.c_int
    lib.gdn_varlen_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int]
    lib.gdn_varlen_bwd_workspace_bytes.restype = sz
    lib.gdn_attn_prefill.argtypes = ([vp] * 6 + [f32] + [vp] * 3 + [i32] * 7
                                     + [f32, ctypes.c_int, vp, sz, vp])
    lib.gdn_attn_prefill.restype = ctypes.c_int
    lib.gdn_attn_decode.argtypes = ([vp] * 6 + [f32] + [vp] * 4 + [i32] * 6
                                    + [f32, ctypes.c_int, vp, sz, vp])
    lib.gdn_attn_decode.restype = ctypes.c_int
    for name in ("gdn_attn_prefill_workspace_bytes", "gdn_attn_decode_workspace_bytes"):
        getattr(lib, name).argtypes = [i32] * 5 + [ctypes.c_int]
        getattr(lib, name).restype = sz
    lib.gdn_status_str.argtypes = [ctypes.c_int]
    lib.gdn_status_str.restype = ctypes.c_char_p
    lib.gdn_last_hip_error.argtypes = []
    lib.gdn_last_hip_error.restype = ctypes.c_int
    lib.gdn_abi_version.argtypes = []
    lib.gdn_abi_version.restype = ctypes.c_int
    return lib


lib = _load()


# ---------------------------------------------------------------- helpers
def status_str(status: int) -> str:
    return lib.gdn_status_str(status).decode()


def last_hip_error() -> int:
    return lib.gdn_last_hip_error()


def abi_version() -> int:
    return lib.gdn_abi_version()


def _check(rc: int, what: str):
    if rc != 0:
        extra = ""
        if rc == -7:
            extra = " (hipError %d)" % last_hip_error()
        raise GDNError(rc, "%s: %s%s" % (what, status_str(rc), extra))


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _req(t, name, dtype=None, ndim=None, device=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def prefill_workspace_bytes(B, T, H_qk, H_v, D=HEAD_DIM, dtype=torch.bfloat16) -> int:
    dt = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    return int(lib.gdn_prefill_workspace_bytes(B, T, H_qk, H_v, D, dt))


def varlen_workspace_bytes(N, T_tot, H_qk, H_v, D=HEAD_DIM, dtype=torch.bfloat16) -> int:
    dt = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    return int(lib.gdn_varlen_workspace_bytes(N, T_tot, H_qk, H_v, D, dt))


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return None
    if workspace is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError("workspace too small: %d < %d bytes" %
                         (workspace.numel() * workspace.element_size(), nbytes))
    return workspace


# ---------------------------------------------------------------- prefill
def _prefill_args(q, k, v, alpha, beta, h0, o, ht, output_final_state, workspace,
                  state_dtype=torch.float32):
    _req(q, "q", ndim=4)
    dtype, dev = q.dtype, q.device
    B, T, H_qk, D = q.shape
    _req(k, "k", dtype, 4, dev)
    _req(v, "v", dtype, 4, dev)
    H_v = v.shape[2]
    if tuple(k.shape) != (B, T, H_qk, D) or tuple(v.shape) != (B, T, H_v, D):
        raise ValueError("q/k [B,T,Hqk,D] and v [B,T,Hv,D] disagree: %s %s %s"
                         % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    for name, t in (("alpha", alpha), ("beta", beta)):
        _req(t, name, torch.float32, 3, dev)
        if tuple(t.shape) != (B, T, H_v):
            raise ValueError("%s must be [B,T,Hv]" % name)
    _req(h0, "h0", state_dtype, 4, dev)
    if h0 is not None and tuple(h0.shape) != (B, H_v, D, D):
        raise ValueError("h0 must be [B,Hv,D,D]")
    if o is None:
        o = torch.empty((B, T, H_v, D), dtype=dtype, device=dev)
    _req(o, "o", dtype, 4, dev)
    if ht is None and output_final_state:
        ht = torch.empty((B, H_v, D, D), dtype=state_dtype, device=dev)
    _req(ht, "ht", state_dtype, 4, dev)
    nbytes = prefill_workspace_bytes(B, T, H_qk, H_v, D, dtype)
    ws = _workspace(nbytes, dev, workspace)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(h0), _ptr(o), _ptr(ht),
            B, T, H_qk, H_v, D, _dt(q), _ptr(ws), nbytes, _stream(dev))
    return args, o, ht, ws


def prefill_chunked(q, k, v, alpha, beta, h0=None, *, o=None, ht=None,
                    output_final_state=True, workspace=None, state_dtype=None):
    """Chunked prefill of B equal-length sequences (gdn_prefill_chunked).
    q, k [B,T,Hqk,128]; v [B,T,Hv,128] (bf16 or fp32); alpha, beta [B,T,Hv]
    fp32; h0 [B,Hv,128,128] or None.  States (h0, ht) are fp32, or bf16
    (gdn_prefill_chunked_bf16_state) when ``state_dtype`` is torch.bfloat16;
    by default the dtype of h0, else of ht, else fp32.  Returns (o, ht)."""
    if state_dtype is None:
        state_dtype = h0.dtype if h0 is not None else (ht.dtype if ht is not None
                                                       else torch.float32)
    if state_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("state_dtype must be torch.float32 or torch.bfloat16")
    args, o, ht, _ = _prefill_args(q, k, v, alpha, beta, h0, o, ht, output_final_state,
                                   workspace, state_dtype)
    if state_dtype == torch.bfloat16:
        _check(lib.gdn_prefill_chunked_bf16_state(*args), "gdn_prefill_chunked_bf16_state")
    else:
        _check(lib.gdn_prefill_chunked(*args), "gdn_prefill_chunked")
    return o, ht


NOALLOC_SCRATCH_BYTES = 128 << 20


def prefill_chunked_noalloc(q, k, v, alpha, beta, h0=None, *, o, ht=None):
    """gdn_prefill_chunked_noalloc: the chunked prefill with the library's
    static scratch array as its workspace (the caller passes o, and ht when the
    final state is wanted: this call allocates nothing).  fp32 states.  Calls
    that overlap on one GPU race on the array."""
    _req(q, "q", ndim=4)
    dtype, dev = q.dtype, q.device
    B, T, H_qk, D = q.shape
    _req(k, "k", dtype, 4, dev)
    _req(v, "v", dtype, 4, dev)
    H_v = v.shape[2]
    if tuple(k.shape) != (B, T, H_qk, D) or tuple(v.shape) != (B, T, H_v, D):
        raise ValueError("q/k [B,T,Hqk,D] and v [B,T,Hv,D] disagree")
    for name, t in (("alpha", alpha), ("beta", beta)):
        _req(t, name, torch.float32, 3, dev)
        if tuple(t.shape) != (B, T, H_v):
            raise ValueError("%s must be [B,T,Hv]" % name)
    _req(h0, "h0", torch.float32, 4, dev)
    _req(o, "o", dtype, 4, dev)
    _req(ht, "ht", torch.float32, 4, dev)
    if tuple(o.shape) != (B, T, H_v, D):
        raise ValueError("o must be [B,T,Hv,D]")
    for name, t in (("h0", h0), ("ht", ht)):
        if t is not None and tuple(t.shape) != (B, H_v, D, D):
            raise ValueError("%s must be [B,Hv,D,D]" % name)
    _check(lib.gdn_prefill_chunked_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(h0), _ptr(o), _ptr(ht),
        B, T, H_qk, H_v, D, _dt(q), _stream(dev)), "gdn_prefill_chunked_noalloc")
    return o, ht


def prefill_bwd_workspace_bytes(B, T, H_qk, H_v, D=HEAD_DIM, dtype=torch.bfloat16) -> int:
    dt = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    return int(lib.gdn_prefill_bwd_workspace_bytes(B, T, H_qk, H_v, D, dt))


def prefill_backward(q, k, v, alpha, beta, do, h0=None, dht=None, *, grads=None,
                     want_dh0=True, workspace=None):
    """Gradients of a chunked prefill (gdn_prefill_chunked_bwd) for
    ``L = sum <do, o> + <dht, ht>``.  Inputs as for :func:`prefill_chunked`
    plus do [B,T,Hv,128] (dtype of q) and dht [B,Hv,128,128] fp32 or None.
    Returns ``(dq, dk, dv, dalpha, dbeta, dh0)``; dq/dk/dv in the dtype of q,
    dalpha/dbeta/dh0 fp32 (dh0 None unless ``want_dh0``).  ``grads`` may hold
    preallocated outputs in that order."""
    _req(q, "q", ndim=4)
    dtype, dev = q.dtype, q.device
    B, T, H_qk, D = q.shape
    _req(k, "k", dtype, 4, dev)
    _req(v, "v", dtype, 4, dev)
    _req(do, "do", dtype, 4, dev)
    H_v = v.shape[2]
    if (tuple(k.shape) != (B, T, H_qk, D) or tuple(v.shape) != (B, T, H_v, D)
            or tuple(do.shape) != (B, T, H_v, D)):
        raise ValueError("q/k [B,T,Hqk,D], v/do [B,T,Hv,D] disagree")
    for name, t in (("alpha", alpha), ("beta", beta)):
        _req(t, name, torch.float32, 3, dev)
        if tuple(t.shape) != (B, T, H_v):
            raise ValueError("%s must be [B,T,Hv]" % name)
    for name, t in (("h0", h0), ("dht", dht)):
        _req(t, name, torch.float32, 4, dev)
        if t is not None and tuple(t.shape) != (B, H_v, D, D):
            raise ValueError("%s must be [B,Hv,D,D]" % name)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                 torch.empty_like(alpha), torch.empty_like(beta),
                 torch.empty((B, H_v, D, D), dtype=torch.float32, device=dev)
                 if want_dh0 else None)
    dq, dk, dv, da, db, dh0 = grads
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _req(t, name, dtype, 4, dev)
        if t.shape != ref.shape:
            raise ValueError("%s must have the shape of its input" % name)
    for name, t in (("dalpha", da), ("dbeta", db)):
        _req(t, name, torch.float32, 3, dev)
        if tuple(t.shape) != (B, T, H_v):
            raise ValueError("%s must be [B,T,Hv]" % name)
    _req(dh0, "dh0", torch.float32, 4, dev)
    nbytes = prefill_bwd_workspace_bytes(B, T, H_qk, H_v, D, dtype)
    ws = _workspace(nbytes, dev, workspace)
    _check(lib.gdn_prefill_chunked_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(h0), _ptr(do), _ptr(dht),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(da), _ptr(db), _ptr(dh0),
        B, T, H_qk, H_v, D, _dt(q), _ptr(ws), nbytes, _stream(dev)), "gdn_prefill_chunked_bwd")
    return dq, dk, dv, da, db, dh0


def varlen_bwd_workspace_bytes(N, T_tot, H_qk, H_v, D=HEAD_DIM, dtype=torch.bfloat16) -> int:
    dt = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    return int(lib.gdn_varlen_bwd_workspace_bytes(N, T_tot, H_qk, H_v, D, dt))


def prefill_varlen_backward(q, k, v, alpha, beta, cu_seqlens, do, h0=None, dht=None, *,
                            want_dh0=True, workspace=None):
    """Gradients of a packed prefill (gdn_prefill_varlen_bwd): q, k [T_tot,
    Hqk, 128]; v, do [T_tot, Hv, 128]; alpha, beta [T_tot, Hv]; cu_seqlens
    int32 [N+1] on the device; h0, dht [N, Hv, 128, 128] fp32 or None.
    Returns (dq, dk, dv, dalpha, dbeta, dh0)."""
    _req(q, "q", ndim=3)
    dtype, dev = q.dtype, q.device
    T_tot, H_qk, D = q.shape
    for name, t in (("k", k), ("v", v), ("do", do)):
        _req(t, name, dtype, 3, dev)
    H_v = v.shape[1]
    if tuple(k.shape) != (T_tot, H_qk, D) or tuple(v.shape) != (T_tot, H_v, D) \
            or tuple(do.shape) != (T_tot, H_v, D):
        raise ValueError("q/k [T,Hqk,D], v/do [T,Hv,D] disagree")
    for name, t in (("alpha", alpha), ("beta", beta)):
        _req(t, name, torch.float32, 2, dev)
        if tuple(t.shape) != (T_tot, H_v):
            raise ValueError("%s must be [T_tot,Hv]" % name)
    _req(cu_seqlens, "cu_seqlens", torch.int32, 1, dev)
    N = cu_seqlens.numel() - 1
    for name, t in (("h0", h0), ("dht", dht)):
        _req(t, name, torch.float32, 4, dev)
        if t is not None and tuple(t.shape) != (N, H_v, D, D):
            raise ValueError("%s must be [N,Hv,D,D]" % name)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    da, db = torch.empty_like(alpha), torch.empty_like(beta)
    dh0 = torch.empty((N, H_v, D, D), dtype=torch.float32, device=dev) if want_dh0 else None
    nbytes = varlen_bwd_workspace_bytes(N, T_tot, H_qk, H_v, D, dtype)
    ws = _workspace(nbytes, dev, workspace)
    _check(lib.gdn_prefill_varlen_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(cu_seqlens), N, T_tot,
        _ptr(h0), _ptr(do), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(da), _ptr(db),
        _ptr(dh0), H_qk, H_v, D, _dt(q), _ptr(ws), nbytes, _stream(dev)),
        "gdn_prefill_varlen_bwd")
    return dq, dk, dv, da, db, dh0


def prefill_prepare(q, k, v, alpha, beta, h0, o, ht, workspace):
    """First half of prefill_chunked (gdn_prefill_prepare): in-chunk solve into
    the workspace.  All buffers are the caller's."""
    args, _, _, _ = _prefill_args(q, k, v, alpha, beta, h0, o, ht, ht is not None, workspace)
    _check(lib.gdn_prefill_prepare(*args), "gdn_prefill_prepare")


def prefill_scan(q, k, v, alpha, beta, h0, o, ht, workspace):
    """Second half of prefill_chunked (gdn_prefill_scan): serial carry and
    outputs, reading what prefill_prepare left in the workspace."""
    args, _, _, _ = _prefill_args(q, k, v, alpha, beta, h0, o, ht, ht is not None, workspace)
    _check(lib.gdn_prefill_scan(*args), "gdn_prefill_scan")


# ---------------------------------------------------------------- decode
def decode_step(q, k, v, alpha, beta, state, *, o=None):
    """One token per sequence; ``state`` [B,Hv,128,128] is updated in place:
    fp32 (gdn_decode_step) or bf16 (gdn_decode_step_bf16_state).  Returns
    o [B,Hv,128]."""
    _req(q, "q", ndim=3)
    dtype, dev = q.dtype, q.device
    B, H_qk, D = q.shape
    _req(k, "k", dtype, 3, dev)
    _req(v, "v", dtype, 3, dev)
    H_v = v.shape[1]
    if tuple(k.shape) != (B, H_qk, D) or tuple(v.shape) != (B, H_v, D):
        raise ValueError("q/k [B,Hqk,D] and v [B,Hv,D] disagree")
    for name, t in (("alpha", alpha), ("beta", beta)):
        _req(t, name, torch.float32, 2, dev)
        if tuple(t.shape) != (B, H_v):
            raise ValueError("%s must be [B,Hv]" % name)
    if not isinstance(state, torch.Tensor) or state.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("state must be a float32 or bfloat16 tensor")
    _req(state, "state", state.dtype, 4, dev)
    if tuple(state.shape) != (B, H_v, D, D):
        raise ValueError("state must be [B,Hv,D,D]")
    if o is None:
        o = torch.empty((B, H_v, D), dtype=dtype, device=dev)
    _req(o, "o", dtype, 3, dev)
    fn = lib.gdn_decode_step if state.dtype == torch.float32 else lib.gdn_decode_step_bf16_state
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state),
            _ptr(o), B, H_qk, H_v, D, _dt(q), _stream(dev))
    _check(rc, "gdn_decode_step")
    return o


def _multi_args(k, v, alpha, beta, state):
    _req(k, "k", ndim=4)
    dtype, dev = k.dtype, k.device
    B, n, H_qk, D = k.shape
    _req(v, "v", dtype, 4, dev)
    H_v = v.shape[2]
    if tuple(v.shape) != (B, n, H_v, D):
        raise ValueError("k [B,n,Hqk,D] and v [B,n,Hv,D] disagree")
    for name, t in (("alpha", alpha), ("beta", beta)):
        _req(t, name, torch.float32, 3, dev)
        if tuple(t.shape) != (B, n, H_v):
            raise ValueError("%s must be [B,n,Hv]" % name)
    _req(state, "state", torch.float32, 4, dev)
    if tuple(state.shape) != (B, H_v, D, D):
        raise ValueError("state must be [B,Hv,D,D]")
    return dtype, dev, B, n, H_qk, H_v, D


def decode_verify(q, k, v, alpha, beta, state, *, o=None):
    """Outputs of n drafted tokens per sequence from ``state`` (not modified)
    (gdn_decode_verify).  q, k [B,n,Hqk,128]; v [B,n,Hv,128]; alpha, beta
    [B,n,Hv] fp32; state [B,Hv,128,128] fp32.  Returns o [B,n,Hv,128]."""
    dtype, dev, B, n, H_qk, H_v, D = _multi_args(k, v, alpha, beta, state)
    _req(q, "q", dtype, 4, dev)
    if tuple(q.shape) != tuple(k.shape):
        raise ValueError("q and k must have the same shape")
    if o is None:
        o = torch.empty((B, n, H_v, D), dtype=dtype, device=dev)
    _req(o, "o", dtype, 4, dev)
    _check(lib.gdn_decode_verify(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                 _ptr(state), _ptr(o), B, n, H_qk, H_v, D, _dt(k), _stream(dev)),
           "gdn_decode_verify")
    return o


def decode_commit(k, v, alpha, beta, state, n_accept):
    """Advance ``state`` in place by the first n_accept[b] drafted tokens of
    each sequence (gdn_decode_commit); n_accept is an int32 tensor [B] on the
    device."""
    dtype, dev, B, n, H_qk, H_v, D = _multi_args(k, v, alpha, beta, state)
    _req(n_accept, "n_accept", torch.int32, 1, dev)
    if n_accept.shape[0] != B:
        raise ValueError("n_accept must be [B]")
    _check(lib.gdn_decode_commit(_ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state),
                                 _ptr(n_accept), B, n, H_qk, H_v, D, _dt(k), _stream(dev)),
           "gdn_decode_commit")


# ---------------------------------------------------------------- varlen
def prefill_varlen(q, k, v, alpha, beta, cu_seqlens, h0=None, *, gate=None,
                   norm_weight=None, norm_eps=1e-6, o=None, ht=None,
                   output_final_state=True, workspace=None):
    """Packed sequences (gdn_prefill_varlen).  q, k [T_tot,Hqk,128]; v, gate
    [T_tot,Hv,128]; alpha, beta [T_tot,Hv]; cu_seqlens int32 [N+1] on the
    device; h0 [N,Hv,128,128] or None.  Returns (o or gated y, ht)."""
    _req(q, "q", ndim=3)
    dtype, dev = q.dtype, q.device
    T_tot, H_qk, D = q.shape
    _req(k, "k", dtype, 3, dev)
    _req(v, "v", dtype, 3, dev)
    H_v = v.shape[1]
    if tuple(k.shape) != (T_tot, H_qk, D) or tuple(v.shape) != (T_tot, H_v, D):
        raise ValueError("q/k [T,Hqk,D] and v [T,Hv,D] disagree")
    for name, t in (("alpha", alpha), ("beta", beta)):
        _req(t, name, torch.float32, 2, dev)
        if tuple(t.shape) != (T_tot, H_v):
            raise ValueError("%s must be [T_tot,Hv]" % name)
    _req(cu_seqlens, "cu_seqlens", torch.int32, 1, dev)
    N = cu_seqlens.shape[0] - 1
    _req(h0, "h0", torch.float32, 4, dev)
    if h0 is not None and tuple(h0.shape) != (N, H_v, D, D):
        raise ValueError("h0 must be [N,Hv,D,D]")
    _req(gate, "gate", dtype, 3, dev)
    if gate is not None and tuple(gate.shape) != (T_tot, H_v, D):
        raise ValueError("gate must be [T_tot,Hv,D]")
    _req(norm_weight, "norm_weight", torch.float32, 1, dev)
    if o is None:
        o = torch.empty((T_tot, H_v, D), dtype=dtype, device=dev)
    _req(o, "o", dtype, 3, dev)
    if ht is None and output_final_state:
        ht = torch.empty((N, H_v, D, D), dtype=torch.float32, device=dev)
    _req(ht, "ht", torch.float32, 4, dev)
    nbytes = varlen_workspace_bytes(N, T_tot, H_qk, H_v, D, dtype)
    ws = _workspace(nbytes, dev, workspace)
    rc = lib.gdn_prefill_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                _ptr(cu_seqlens), N, T_tot, _ptr(h0), _ptr(o), _ptr(ht),
                                _ptr(gate), _ptr(norm_weight), float(norm_eps), H_qk, H_v, D,
                                _dt(q), _ptr(ws), nbytes, _stream(dev))
    _check(rc, "gdn_prefill_varlen")
    return o, ht


# ---------------------------------------------------------------- gated attention
ATTN_DIM = 256


def _attn_common(q, k, v, gate, q_norm_w, k_norm_w, lead):
    _req(q, "q", ndim=len(lead) + 2)
    dtype, dev = q.dtype, q.device
    Hq, D = q.shape[-2], q.shape[-1]
    Hkv = k.shape[-2]
    for name, t, H in (("k", k, Hkv), ("v", v, Hkv), ("gate", gate, Hq)):
        _req(t, name, dtype, len(lead) + 2, dev)
        if tuple(t.shape) != tuple(lead) + (H, D):
            raise ValueError("%s must be %s" % (name, tuple(lead) + (H, D)))
    for name, t in (("q_norm_w", q_norm_w), ("k_norm_w", k_norm_w)):
        _req(t, name, torch.float32, 1, dev)
    return dtype, dev, Hq, Hkv, D


def attn_prefill_workspace_bytes(B, T, H_q=24, H_kv=4, D=ATTN_DIM, dtype=torch.bfloat16) -> int:
    dt = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    return int(lib.gdn_attn_prefill_workspace_bytes(B, T, H_q, H_kv, D, dt))


def attn_decode_workspace_bytes(B, cache_len, H_q=24, H_kv=4, D=ATTN_DIM,
                                dtype=torch.bfloat16) -> int:
    dt = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    return int(lib.gdn_attn_decode_workspace_bytes(B, cache_len, H_q, H_kv, D, dt))


def attn_prefill(q, k, v, gate, q_norm_w=None, k_norm_w=None, *, eps=1e-6, rope_dim=64,
                 theta=1.0e7, k_cache=None, v_cache=None, o=None, workspace=None):
    """Gated attention of a prefill (gdn_attn_prefill).  q, gate [B,T,Hq,256];
    k, v [B,T,Hkv,256]; optional caches [B,cache_len,Hkv,256] receive the
    normalised, rotated keys and the values of positions 0..T-1.  Returns o."""
    B, T = q.shape[0], q.shape[1]
    dtype, dev, Hq, Hkv, D = _attn_common(q, k, v, gate, q_norm_w, k_norm_w, (B, T))
    cache_len = 0
    if k_cache is not None or v_cache is not None:
        _req(k_cache, "k_cache", dtype, 4, dev)
        _req(v_cache, "v_cache", dtype, 4, dev)
        cache_len = k_cache.shape[1]
    if o is None:
        o = torch.empty_like(q)
    _req(o, "o", dtype, 4, dev)
    nbytes = attn_prefill_workspace_bytes(B, T, Hq, Hkv, D, dtype)
    ws = _workspace(nbytes, dev, workspace)
    _check(lib.gdn_attn_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(q_norm_w), _ptr(k_norm_w), eps, _ptr(o),
        _ptr(k_cache), _ptr(v_cache), cache_len, B, T, Hq, Hkv, D, rope_dim, theta, _dt(q),
        _ptr(ws), nbytes, _stream(dev)), "gdn_attn_prefill")
    return o


def attn_decode(q, k, v, gate, k_cache, v_cache, pos, q_norm_w=None, k_norm_w=None, *,
                eps=1e-6, rope_dim=64, theta=1.0e7, o=None, workspace=None):
    """One decode token per sequence (gdn_attn_decode).  q, gate [B,Hq,256];
    k, v [B,Hkv,256]; caches [B,cache_len,Hkv,256]; pos int32 [B] on the
    device (tokens already cached).  Writes the token's key/value at pos and
    returns o [B,Hq,256]."""
    B = q.shape[0]
    dtype, dev, Hq, Hkv, D = _attn_common(q, k, v, gate, q_norm_w, k_norm_w, (B,))
    _req(k_cache, "k_cache", dtype, 4, dev)
    _req(v_cache, "v_cache", dtype, 4, dev)
    _req(pos, "pos", torch.int32, 1, dev)
    cache_len = k_cache.shape[1]
    if o is None:
        o = torch.empty_like(q)
    _req(o, "o", dtype, 3, dev)
    nbytes = attn_decode_workspace_bytes(B, cache_len, Hq, Hkv, D, dtype)
    ws = _workspace(nbytes, dev, workspace)
    _check(lib.gdn_attn_decode(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(q_norm_w), _ptr(k_norm_w), eps, _ptr(o),
        _ptr(k_cache), _ptr(v_cache), _ptr(pos), cache_len, B, Hq, Hkv, D, rope_dim, theta,
        _dt(q), _ptr(ws), nbytes, _stream(dev)), "gdn_attn_decode")
    return o


# ---------------------------------------------------------------- autograd
class GatedDeltaRule(torch.autograd.Function):
    """The chunked prefill as a differentiable op: forward is
    gdn_prefill_chunked, backward is gdn_prefill_chunked_bwd (which
    recomputes the forward states; nothing but the inputs is saved).

    ``o, ht = GatedDeltaRule.apply(q, k, v, alpha, beta, h0)``; h0 may be None.
    Gradients flow to q, k, v, alpha, beta and h0."""

    @staticmethod
    def forward(ctx, q, k, v, alpha, beta, h0):
        o, ht = prefill_chunked(q, k, v, alpha, beta, h0)
        ctx.save_for_backward(q, k, v, alpha, beta, h0)
        ctx.has_h0 = h0 is not None
        return o, ht

    @staticmethod
    def backward(ctx, do, dht):
        q, k, v, alpha, beta, h0 = ctx.saved_tensors
        if do is None:
            do = torch.zeros((q.shape[0], q.shape[1], v.shape[2], v.shape[3]), dtype=q.dtype,
                             device=q.device)
        dq, dk, dv, da, db, dh0 = prefill_backward(
            q, k, v, alpha, beta, do.contiguous(), h0 if ctx.has_h0 else None,
            None if dht is None else dht.contiguous(), want_dh0=ctx.has_h0)
        return dq, dk, dv, da, db, dh0


def gated_delta_rule(q, k, v, alpha, beta, h0=None):
    """Differentiable chunked prefill: returns (o, ht)."""
    return GatedDeltaRule.apply(q, k, v, alpha, beta, h0)
