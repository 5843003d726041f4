"""Thin ctypes binding of libgma.so (declared in include/gma.h).

Argument marshalling only: every step of the forward runs in the library's HIP
kernels.  PyTorch supplies device memory (``torch.empty``) and the current HIP
stream (``torch.cuda.current_stream().cuda_stream``).  If the library is missing
or cannot be loaded every call raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgma.so")

GMA_OK = 0
GMA_F32, GMA_BF16 = 0, 1
ALGO = {"auto": 0, "simt": 1, "mfma": 2}

_lib = None


class GMAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"gma error {code}: {msg}")
        self.code = code


class GmaDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d_r", ctypes.c_int32), ("d_v", ctypes.c_int32), ("K", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("algo", ctypes.c_int32), ("var_floor", ctypes.c_float)]


def load_library(path: Optional[str] = None):
    """Load libgma.so (built in-tree by ``gaussian_mixture_sequence_resp_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    # torch ships its own HIP runtime (SONAME libamdhip64.so.7); loading torch first makes
    # libgma.so bind to that same runtime instead of pulling in a second copy.
    import torch  # noqa: F401
    if not os.path.exists(p):
        raise GMAError(-100, f"HIP library not built: {p} is missing "
                             "(run __graft_entry__.build() or python -m "
                             "gaussian_mixture_sequence_resp_amd.build)")
    lib = ctypes.CDLL(p)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.gma_workspace_size.argtypes = [ctypes.POINTER(GmaDesc), ctypes.c_int]
    lib.gma_workspace_size.restype = sz
    lib.gma_forward.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_float, vp, vp,
                                ctypes.POINTER(GmaDesc), vp, sz, vp]
    lib.gma_forward.restype = ctypes.c_int
    lib.gma_forward_timed.argtypes = lib.gma_forward.argtypes + [
        ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
        ctypes.POINTER(ctypes.c_int)]
    lib.gma_forward_timed.restype = ctypes.c_int
    lib.gma_workspace_size_cross.argtypes = [ctypes.POINTER(GmaDesc), ctypes.c_int32]
    lib.gma_workspace_size_cross.restype = sz
    lib.gma_forward_cross.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int32, ctypes.c_float, vp, vp,
                                      ctypes.POINTER(GmaDesc), vp, sz, vp]
    lib.gma_forward_cross.restype = ctypes.c_int
    lib.gma_forward_cross_timed.argtypes = lib.gma_forward_cross.argtypes + [
        ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
        ctypes.POINTER(ctypes.c_int)]
    lib.gma_forward_cross_timed.restype = ctypes.c_int
    lib.gma_memory_workspace_size.argtypes = [ctypes.POINTER(GmaDesc)]
    lib.gma_memory_workspace_size.restype = sz
    lib.gma_memory.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(GmaDesc), vp, sz, vp]
    lib.gma_memory.restype = ctypes.c_int
    lib.gma_decode_workspace_size.argtypes = [ctypes.POINTER(GmaDesc)]
    lib.gma_decode_workspace_size.restype = sz
    lib.gma_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, ctypes.POINTER(GmaDesc), vp,
                                    sz, vp]
    lib.gma_decode_step.restype = ctypes.c_int
    lib.gma_decode_prepared_size.argtypes = [ctypes.POINTER(GmaDesc)]
    lib.gma_decode_prepared_size.restype = sz
    lib.gma_decode_prepare.argtypes = [vp, vp, vp, vp, sz, ctypes.POINTER(GmaDesc), vp]
    lib.gma_decode_prepare.restype = ctypes.c_int
    lib.gma_decode_step_prepared.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp, ctypes.POINTER(GmaDesc), vp]
    lib.gma_decode_step_prepared.restype = ctypes.c_int
    lib.gma_backward_workspace_size.argtypes = [ctypes.POINTER(GmaDesc), ctypes.c_int]
    lib.gma_backward_workspace_size.restype = sz
    lib.gma_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_float, vp, vp, vp, vp, vp, vp,
                                 ctypes.POINTER(GmaDesc), vp, sz, vp]
    lib.gma_backward.restype = ctypes.c_int
    lib.gma_stats_workspace_size.argtypes = [ctypes.POINTER(GmaDesc)]
    lib.gma_stats_workspace_size.restype = sz
    lib.gma_resp_stats.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(GmaDesc), vp, sz, vp]
    lib.gma_resp_stats.restype = ctypes.c_int
    lib.gma_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_float, vp, vp,
                                        ctypes.POINTER(GmaDesc), vp]
    lib.gma_forward_noalloc.restype = ctypes.c_int
    lib.gma_strerror.argtypes = [ctypes.c_int]
    lib.gma_strerror.restype = ctypes.c_char_p
    lib.gma_version.argtypes = []
    lib.gma_version.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def strerror(code: int) -> str:
    return load_library().gma_strerror(int(code)).decode()


def version() -> int:
    return int(load_library().gma_version())


def make_desc(B, H, N, d_r, d_v, K, dtype: str, var_floor: float, algo: str = "auto") -> GmaDesc:
    dt = {"f32": GMA_F32, "bf16": GMA_BF16}[dtype]
    return GmaDesc(int(B), int(H), int(N), int(d_r), int(d_v), int(K), dt, ALGO[algo],
                   float(var_floor))


def workspace_size(desc: GmaDesc, causal: bool) -> int:
    return int(load_library().gma_workspace_size(ctypes.byref(desc), 1 if causal else 0))


def workspace_size_cross(desc: GmaDesc, n_k: int) -> int:
    return int(load_library().gma_workspace_size_cross(ctypes.byref(desc), int(n_k)))


def _dense(*ts):
    """The C ABI takes dense row-major tensors: refuse strided views (a silent misread
    otherwise)."""
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise GMAError(-2, f"tensor of shape {tuple(t.shape)} is not contiguous (call .contiguous())")


def _dtype_name(t) -> str:
    import torch
    if t.dtype == torch.float32:
        return "f32"
    if t.dtype == torch.bfloat16:
        return "bf16"
    raise GMAError(-3, f"unsupported dtype {t.dtype}")


GMA_ERR_DEVICE = -101  # binding only: a tensor is not on the GPU that holds qr (or x)


def _check(specs, device_of):
    """Validate every tensor argument before any library call: ``specs`` lists
    (name, tensor, expected shape or None for any, expected torch dtype or None, required).
    Shapes and dtypes are checked first (status -2 / -3, as the library would report for
    its own descriptor), then that every tensor lives on the CUDA device of ``device_of``
    (-101): a host pointer or another device's memory would be read by the kernels."""
    for name, t, shape, dtype, required in specs:
        if t is None:
            if required:
                raise GMAError(-1, f"{name} is required")
            continue
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise GMAError(-2, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if dtype is not None and t.dtype != dtype:
            raise GMAError(-3, f"{name} has dtype {t.dtype}, expected {dtype}")
    dev = device_of.device
    if dev.type != "cuda":
        raise GMAError(GMA_ERR_DEVICE, f"tensors must be on a GPU (got {dev})")
    for name, t, _, _, _ in specs:
        if t is not None and t.device != dev:
            raise GMAError(GMA_ERR_DEVICE, f"{name} is on {t.device}, expected {dev}")


def _need4(name, t):
    if t.dim() != 4:
        raise GMAError(-2, f"{name} must be 4-D, got shape {tuple(t.shape)}")


def _params_specs(H, K, d_r, mu, var_raw, prior_logits):
    import torch
    return [("mu", mu, (H, K, d_r), torch.float32, True),
            ("var_raw", var_raw, (H, K, d_r), torch.float32, True),
            ("prior_logits", prior_logits, (H, K), torch.float32, True)]


def _ws_spec(workspace):
    import torch
    return [("workspace", workspace, None, torch.uint8, False)]


def forward(qr, kr, v, mu, var_raw, prior_logits, causal: bool = False, eps: float = 1e-6,
            var_floor: float = 1e-3, out=None, gamma_out=None, workspace=None,
            algo: str = "auto", stream=None, events=None, names=None):
    """GMA forward on the current HIP device.

    qr, kr [B,H,N,d_r] and v [B,H,N,d_v] (float32 or bfloat16, contiguous, on the GPU);
    mu, var_raw [H,K,d_r] and prior_logits [H,K] float32.  Returns ``out`` [B,H,N,d_v] in
    the input dtype.  ``gamma_out`` (optional, float32 [2,B,H,N,K]) receives Gamma_Q and
    Gamma_K.  ``workspace`` (optional, uint8 device tensor) is allocated if not given.
    """
    import torch
    _need4("qr", qr)
    _need4("v", v)
    B, H, N, d_r = qr.shape
    d_v = v.shape[-1]
    if mu.dim() != 3:
        raise GMAError(-2, f"mu must be [H, K, d_r], got shape {tuple(mu.shape)}")
    K = mu.shape[1]
    dt = _dtype_name(qr)
    _check([("qr", qr, None, None, True), ("kr", kr, (B, H, N, d_r), qr.dtype, True),
            ("v", v, (B, H, N, d_v), qr.dtype, True)]
           + _params_specs(H, K, d_r, mu, var_raw, prior_logits)
           + [("out", out, (B, H, N, d_v), qr.dtype, False),
              ("gamma_out", gamma_out, (2, B, H, N, K), torch.float32, False)] + _ws_spec(workspace), qr)
    _dense(qr, kr, v, mu, var_raw, prior_logits, out, gamma_out)
    lib = load_library()
    desc = make_desc(B, H, N, d_r, d_v, K, dt, var_floor, algo)
    if out is None:
        out = torch.empty((B, H, N, d_v), dtype=qr.dtype, device=qr.device)
    need = int(lib.gma_workspace_size(ctypes.byref(desc), 1 if causal else 0))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=qr.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream(qr.device).cuda_stream

    def ptr(t):
        return None if t is None else t.data_ptr()

    args = (ptr(qr), ptr(kr), ptr(v), ptr(mu), ptr(var_raw), ptr(prior_logits),
            1 if causal else 0, float(eps), ptr(out), ptr(gamma_out),
            ctypes.byref(desc), ws_ptr, ws_bytes, stream)
    if events is None:
        st = lib.gma_forward(*args)
    else:
        # events: ctypes array of hipEvent_t handles; names: ctypes array of c_char_p
        nk = ctypes.c_int(0)
        st = lib.gma_forward_timed(*args, events, len(events), names, ctypes.byref(nk))
        forward.last_kernel_count = nk.value
    if st != GMA_OK:
        raise GMAError(st, strerror(st))
    return out


def forward_noalloc(qr, kr, v, mu, var_raw, prior_logits, out, causal: bool = False, eps: float = 1e-6,
                    var_floor: float = 1e-3, gamma_out=None, algo: str = "auto", stream=None):
    """gma_forward_noalloc: the forward with the library's static scratch (no workspace,
    nothing allocated by the call).  ``out`` [B,H,N,d_v] must be given (preallocated)."""
    import torch
    _need4("qr", qr)
    _need4("v", v)
    B, H, N, d_r = qr.shape
    d_v = v.shape[-1]
    if mu.dim() != 3:
        raise GMAError(-2, f"mu must be [H, K, d_r], got shape {tuple(mu.shape)}")
    K = mu.shape[1]
    dt = _dtype_name(qr)
    _check([("qr", qr, None, None, True), ("kr", kr, (B, H, N, d_r), qr.dtype, True),
            ("v", v, (B, H, N, d_v), qr.dtype, True)]
           + _params_specs(H, K, d_r, mu, var_raw, prior_logits)
           + [("out", out, (B, H, N, d_v), qr.dtype, True),
              ("gamma_out", gamma_out, (2, B, H, N, K), torch.float32, False)], qr)
    _dense(qr, kr, v, mu, var_raw, prior_logits, out, gamma_out)
    lib = load_library()
    desc = make_desc(B, H, N, d_r, d_v, K, dt, var_floor, algo)
    if stream is None:
        stream = torch.cuda.current_stream(qr.device).cuda_stream
    st = lib.gma_forward_noalloc(qr.data_ptr(), kr.data_ptr(), v.data_ptr(), mu.data_ptr(), var_raw.data_ptr(),
                                 prior_logits.data_ptr(), 1 if causal else 0, float(eps), out.data_ptr(),
                                 None if gamma_out is None else gamma_out.data_ptr(), ctypes.byref(desc), stream)
    if st != GMA_OK:
        raise GMAError(st, strerror(st))
    return out


def forward_cross(qr, kr, v, mu, var_raw, prior_logits, eps: float = 1e-6, var_floor: float = 1e-3,
                  out=None, gamma_out=None, workspace=None, algo: str = "auto", stream=None,
                  events=None, names=None):
    """Cross variant (bidirectional): qr [B,H,Nq,d_r]; kr [B,H,Nk,d_r]; v [B,H,Nk,d_v].
    Returns ``out`` [B,H,Nq,d_v].  ``gamma_out`` (optional, float32, B*H*(Nq+Nk)*K
    elements) receives Gamma_Q [B,H,Nq,K] followed by Gamma_K [B,H,Nk,K]."""
    import torch
    _need4("qr", qr)
    _need4("kr", kr)
    _need4("v", v)
    B, H, Nq, d_r = qr.shape
    Nk = kr.shape[2]
    d_v = v.shape[-1]
    if mu.dim() != 3:
        raise GMAError(-2, f"mu must be [H, K, d_r], got shape {tuple(mu.shape)}")
    K = mu.shape[1]
    dt = _dtype_name(qr)
    gamma_shape = None if gamma_out is None else (gamma_out.numel(),)
    if gamma_out is not None and gamma_out.numel() != B * H * (Nq + Nk) * K:
        raise GMAError(-2, f"gamma_out has {gamma_out.numel()} elements, expected {B * H * (Nq + Nk) * K}")
    _check([("qr", qr, None, None, True), ("kr", kr, (B, H, Nk, d_r), qr.dtype, True),
            ("v", v, (B, H, Nk, d_v), qr.dtype, True)]
           + _params_specs(H, K, d_r, mu, var_raw, prior_logits)
           + [("out", out, (B, H, Nq, d_v), qr.dtype, False),
              ("gamma_out", None if gamma_out is None else gamma_out.reshape(-1), gamma_shape, torch.float32,
               False)] + _ws_spec(workspace), qr)
    _dense(qr, kr, v, mu, var_raw, prior_logits, out, gamma_out)
    lib = load_library()
    desc = make_desc(B, H, Nq, d_r, d_v, K, dt, var_floor, algo)
    if out is None:
        out = torch.empty((B, H, Nq, d_v), dtype=qr.dtype, device=qr.device)
    need = int(lib.gma_workspace_size_cross(ctypes.byref(desc), Nk))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=qr.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream(qr.device).cuda_stream

    def ptr(t):
        return None if t is None else t.data_ptr()

    args = (ptr(qr), ptr(kr), ptr(v), ptr(mu), ptr(var_raw), ptr(prior_logits), int(Nk), float(eps),
            ptr(out), ptr(gamma_out), ctypes.byref(desc), ws_ptr, ws_bytes, stream)
    if events is None:
        st = lib.gma_forward_cross(*args)
    else:
        nk = ctypes.c_int(0)
        st = lib.gma_forward_cross_timed(*args, events, len(events), names, ctypes.byref(nk))
        forward_cross.last_kernel_count = nk.value
    if st != GMA_OK:
        raise GMAError(st, strerror(st))
    return out


def _ws(need, like):
    import torch
    return torch.empty(max(need, 1), dtype=torch.uint8, device=like.device)


def memory(kr, v, mu, var_raw, prior_logits, var_floor: float = 1e-3, state=None, workspace=None,
           algo: str = "auto", stream=None):
    """Causal memory [S | z] of the N positions of kr [B,H,N,d_r], v [B,H,N,d_v]:
    returns ``state`` float32 [B,H,K,d_v+1] (row k: S[k, :d_v], z[k])."""
    import torch
    _need4("kr", kr)
    _need4("v", v)
    B, H, N, d_r = kr.shape
    d_v = v.shape[-1]
    if mu.dim() != 3:
        raise GMAError(-2, f"mu must be [H, K, d_r], got shape {tuple(mu.shape)}")
    K = mu.shape[1]
    dt = _dtype_name(kr)
    _check([("kr", kr, None, None, True), ("v", v, (B, H, N, d_v), kr.dtype, True)]
           + _params_specs(H, K, d_r, mu, var_raw, prior_logits)
           + [("state", state, (B, H, K, d_v + 1), torch.float32, False)] + _ws_spec(workspace), kr)
    _dense(kr, v, mu, var_raw, prior_logits, state)
    lib = load_library()
    desc = make_desc(B, H, N, d_r, d_v, K, dt, var_floor, algo)
    if state is None:
        state = torch.empty((B, H, K, d_v + 1), dtype=torch.float32, device=kr.device)
    need = int(lib.gma_memory_workspace_size(ctypes.byref(desc)))
    if workspace is None:
        workspace = _ws(need, kr)
    if stream is None:
        stream = torch.cuda.current_stream(kr.device).cuda_stream
    nz = N > 0
    st = lib.gma_memory(kr.data_ptr() if nz else None, v.data_ptr() if nz else None, mu.data_ptr(),
                        var_raw.data_ptr(), prior_logits.data_ptr(), state.data_ptr(), ctypes.byref(desc),
                        workspace.data_ptr(), workspace.numel(), stream)
    if st != GMA_OK:
        raise GMAError(st, strerror(st))
    return state


def decode_step(qr, kr, v, mu, var_raw, prior_logits, state, eps: float = 1e-6, var_floor: float = 1e-3,
                out=None, workspace=None, algo: str = "auto", stream=None):
    """One causal decode step: qr, kr [B,H,1,d_r] (or [B,H,d_r]), v [B,H,1,d_v] (or [B,H,d_v]);
    ``state`` float32 [B,H,K,d_v+1] is updated in place; returns out [B,H,1,d_v]."""
    import torch
    if qr.dim() not in (3, 4) or (qr.dim() == 4 and qr.shape[2] != 1):
        raise GMAError(-2, f"qr must be [B, H, 1, d_r] or [B, H, d_r], got shape {tuple(qr.shape)}")
    B, H = qr.shape[0], qr.shape[1]
    d_r, d_v = qr.shape[-1], v.shape[-1]
    if mu.dim() != 3:
        raise GMAError(-2, f"mu must be [H, K, d_r], got shape {tuple(mu.shape)}")
    K = mu.shape[1]
    dt = _dtype_name(qr)
    row = (lambda t: None if t is None else t.reshape(t.shape[0], t.shape[1], -1) if t.dim() in (3, 4) else t)
    if kr.dim() not in (3, 4) or v.dim() not in (3, 4):
        raise GMAError(-2, "kr and v must be [B, H, 1, d] or [B, H, d]")
    _check([("qr", row(qr), None, None, True), ("kr", row(kr), (B, H, d_r), qr.dtype, True),
            ("v", row(v), (B, H, d_v), qr.dtype, True)]
           + _params_specs(H, K, d_r, mu, var_raw, prior_logits)
           + [("state", state, (B, H, K, d_v + 1), torch.float32, True),
              ("out", out, (B, H, 1, d_v), qr.dtype, False)] + _ws_spec(workspace), qr)
    qr, kr, v = qr.contiguous(), kr.contiguous(), v.contiguous()  # one row per (b, h): cheap
    _dense(mu, var_raw, prior_logits, state, out)
    lib = load_library()
    desc = make_desc(B, H, 1, d_r, d_v, K, dt, var_floor, algo)
    if out is None:
        out = torch.empty((B, H, 1, d_v), dtype=qr.dtype, device=qr.device)
    need = int(lib.gma_decode_workspace_size(ctypes.byref(desc)))
    if workspace is None and need > 0:
        workspace = _ws(need, qr)
    ws_ptr, ws_bytes = (workspace.data_ptr(), workspace.numel()) if workspace is not None else (None, 0)
    if stream is None:
        stream = torch.cuda.current_stream(qr.device).cuda_stream
    st = lib.gma_decode_step(qr.data_ptr(), kr.data_ptr(), v.data_ptr(), mu.data_ptr(), var_raw.data_ptr(),
                             prior_logits.data_ptr(), state.data_ptr(), float(eps), out.data_ptr(),
                             ctypes.byref(desc), ws_ptr, ws_bytes, stream)
    if st != GMA_OK:
        raise GMAError(st, strerror(st))
    return out


class DecodeParams:
    """Prepared mixture parameters of the decode step (gma_decode_prepare): ``block`` is the
    opaque uint8 device tensor, valid for heads H, K components, d_r routing dims and the
    input dtype it was prepared for."""

    def __init__(self, block, H: int, K: int, d_r: int, dtype: str, var_floor: float):
        self.block, self.H, self.K, self.d_r, self.dtype, self.var_floor = block, H, K, d_r, dtype, var_floor


def decode_prepare(mu, var_raw, prior_logits, dtype: str = "bf16", var_floor: float = 1e-3,
                   stream=None) -> DecodeParams:
    """Prepare mu, var_raw [H,K,d_r] and prior_logits [H,K] (float32, on the GPU) for
    ``decode_step_prepared`` on inputs of ``dtype`` ("f32" or "bf16")."""
    import torch
    if mu.dim() != 3:
        raise GMAError(-2, f"mu must be [H, K, d_r], got shape {tuple(mu.shape)}")
    if dtype not in ("f32", "bf16"):
        raise GMAError(-3, f"unsupported dtype {dtype!r}")
    H, K, d_r = mu.shape
    _check(_params_specs(H, K, d_r, mu, var_raw, prior_logits), mu)
    _dense(mu, var_raw, prior_logits)
    lib = load_library()
    desc = make_desc(1, H, 1, d_r, 1, K, dtype, var_floor)
    need = int(lib.gma_decode_prepared_size(ctypes.byref(desc)))
    if need == 0:
        raise GMAError(-3, f"decode parameters not supported for H={H}, K={K}, d_r={d_r}")
    block = torch.empty(need, dtype=torch.uint8, device=mu.device)
    if stream is None:
        stream = torch.cuda.current_stream(mu.device).cuda_stream
    st = lib.gma_decode_prepare(mu.data_ptr(), var_raw.data_ptr(), prior_logits.data_ptr(), block.data_ptr(),
                                need, ctypes.byref(desc), stream)
    if st != GMA_OK:
        raise GMAError(st, strerror(st))
    return DecodeParams(block, H, K, d_r, dtype, var_floor)


def decode_step_prepared(qr, kr, v, params: DecodeParams, state, eps: float = 1e-6, out=None, stream=None):
    """``decode_step`` on prepared parameters: qr, kr [B,H,1,d_r] (or [B,H,d_r]), v [B,H,1,d_v]
    (or [B,H,d_v]); ``state`` float32 [B,H,K,d_v+1] is updated in place; returns out [B,H,1,d_v]."""
    import torch
    if qr.dim() not in (3, 4) or (qr.dim() == 4 and qr.shape[2] != 1):
        raise GMAError(-2, f"qr must be [B, H, 1, d_r] or [B, H, d_r], got shape {tuple(qr.shape)}")
    if kr.dim() not in (3, 4) or v.dim() not in (3, 4):
        raise GMAError(-2, "kr and v must be [B, H, 1, d] or [B, H, d]")
    B, H = qr.shape[0], qr.shape[1]
    d_r, d_v = qr.shape[-1], v.shape[-1]
    dt = _dtype_name(qr)
    if (H, d_r, dt) != (params.H, params.d_r, params.dtype):
        raise GMAError(-2, f"prepared parameters are for H={params.H}, d_r={params.d_r}, {params.dtype}; "
                           f"got H={H}, d_r={d_r}, {dt}")
    K = params.K
    row = (lambda t: None if t is None else t.reshape(t.shape[0], t.shape[1], -1))
    _check([("qr", row(qr), None, None, True), ("kr", row(kr), (B, H, d_r), qr.dtype, True),
            ("v", row(v), (B, H, d_v), qr.dtype, True), ("prepared", params.block, None, torch.uint8, True),
            ("state", state, (B, H, K, d_v + 1), torch.float32, True),
            ("out", out, (B, H, 1, d_v), qr.dtype, False)], qr)
    qr, kr, v = qr.contiguous(), kr.contiguous(), v.contiguous()
    _dense(state, out)
    lib = load_library()
    desc = make_desc(B, H, 1, d_r, d_v, K, dt, params.var_floor)
    if out is None:
        out = torch.empty((B, H, 1, d_v), dtype=qr.dtype, device=qr.device)
    if stream is None:
        stream = torch.cuda.current_stream(qr.device).cuda_stream
    st = lib.gma_decode_step_prepared(qr.data_ptr(), kr.data_ptr(), v.data_ptr(), params.block.data_ptr(),
                                      state.data_ptr(), float(eps), out.data_ptr(), ctypes.byref(desc), stream)
    if st != GMA_OK:
        raise GMAError(st, strerror(st))
    return out


def resp_stats(x, mu, var_raw, prior_logits, var_floor: float = 1e-3, with_hard: bool = True,
               workspace=None, algo: str = "auto", stream=None) -> dict:
    """Responsibility statistics of the routing rows x [B,H,N,d_r] per head (pooled over
    the batch and the positions): ``hard`` int32 [B,H,N] (argmax, lowest index on ties; only
    with ``with_hard``), ``counts`` int32 [H,K], ``usage`` float32 [H,K], ``used`` int32 [H],
    ``entropy`` float32 [H] (hard-usage entropy over ln K)."""
    import torch
    _need4("x", x)
    B, H, N, d_r = x.shape
    if mu.dim() != 3:
        raise GMAError(-2, f"mu must be [H, K, d_r], got shape {tuple(mu.shape)}")
    K = mu.shape[1]
    dt = _dtype_name(x)
    _check([("x", x, None, None, True)] + _params_specs(H, K, d_r, mu, var_raw, prior_logits) + _ws_spec(workspace),
           x)
    _dense(x, mu, var_raw, prior_logits)
    lib = load_library()
    dev = x.device
    desc = make_desc(B, H, N, d_r, 1, K, dt, var_floor, algo)
    res = {
        "hard": torch.empty((B, H, N), dtype=torch.int32, device=dev) if with_hard else None,
        "counts": torch.empty((H, K), dtype=torch.int32, device=dev),
        "usage": torch.empty((H, K), dtype=torch.float32, device=dev),
        "used": torch.empty((H,), dtype=torch.int32, device=dev),
        "entropy": torch.empty((H,), dtype=torch.float32, device=dev),
    }
    need = int(lib.gma_stats_workspace_size(ctypes.byref(desc)))
    if workspace is None and need > 0:
        workspace = _ws(need, x)
    ws_ptr, ws_bytes = (workspace.data_ptr(), workspace.numel()) if workspace is not None else (None, 0)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    hard = res["hard"].data_ptr() if with_hard else None
    st = lib.gma_resp_stats(x.data_ptr() if N > 0 else None, mu.data_ptr(), var_raw.data_ptr(),
                            prior_logits.data_ptr(), hard, res["counts"].data_ptr(), res["usage"].data_ptr(),
                            res["used"].data_ptr(), res["entropy"].data_ptr(), ctypes.byref(desc), ws_ptr, ws_bytes,
                            stream)
    if st != GMA_OK:
        raise GMAError(st, strerror(st))
    return res


def backward(qr, kr, v, mu, var_raw, prior_logits, dout, causal: bool, eps: float = 1e-6, var_floor: float = 1e-3,
             workspace=None, algo: str = "auto", stream=None) -> dict:
    """Gradients of L = sum(dout * O) for gma_forward: ``dqr``, ``dkr``, ``dv`` (input dtype,
    shapes of qr, kr, v) and ``dmu``, ``dvar_raw`` [H,K,d_r], ``dprior`` [H,K] (float32)."""
    import torch
    _need4("qr", qr)
    _need4("v", v)
    B, H, N, d_r = qr.shape
    d_v = v.shape[-1]
    if mu.dim() != 3:
        raise GMAError(-2, f"mu must be [H, K, d_r], got shape {tuple(mu.shape)}")
    K = mu.shape[1]
    dt = _dtype_name(qr)
    _check([("qr", qr, None, None, True), ("kr", kr, (B, H, N, d_r), qr.dtype, True),
            ("v", v, (B, H, N, d_v), qr.dtype, True)]
           + _params_specs(H, K, d_r, mu, var_raw, prior_logits)
           + [("dout", dout, (B, H, N, d_v), qr.dtype, True)] + _ws_spec(workspace), qr)
    _dense(qr, kr, v, mu, var_raw, prior_logits, dout)
    lib = load_library()
    desc = make_desc(B, H, N, d_r, d_v, K, dt, var_floor, algo)
    g = {"dqr": torch.empty_like(qr), "dkr": torch.empty_like(kr), "dv": torch.empty_like(v),
         "dmu": torch.empty_like(mu), "dvar_raw": torch.empty_like(var_raw), "dprior": torch.empty_like(prior_logits)}
    need = int(lib.gma_backward_workspace_size(ctypes.byref(desc), 1 if causal else 0))
    if workspace is None and need > 0:
        workspace = _ws(need, qr)
    ws_ptr, ws_bytes = (workspace.data_ptr(), workspace.numel()) if workspace is not None else (None, 0)
    if stream is None:
        stream = torch.cuda.current_stream(qr.device).cuda_stream
    ptr = (lambda t: t.data_ptr() if t.numel() else None)
    st = lib.gma_backward(ptr(qr), ptr(kr), ptr(v), mu.data_ptr(), var_raw.data_ptr(), prior_logits.data_ptr(),
                          ptr(dout), 1 if causal else 0, float(eps), ptr(g["dqr"]), ptr(g["dkr"]), ptr(g["dv"]),
                          g["dmu"].data_ptr(), g["dvar_raw"].data_ptr(), g["dprior"].data_ptr(), ctypes.byref(desc),
                          ws_ptr, ws_bytes, stream)
    if st != GMA_OK:
        raise GMAError(st, strerror(st))
    return g
