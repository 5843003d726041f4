"""ctypes front end of the plain-C fp64 oracle (``gma_oracle.c``).

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the product path.

Inputs may be numpy arrays or CPU torch tensors of any float dtype; they are
up-cast exactly to float64 (bf16 and fp32 values are exactly representable) and
made contiguous before the call.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gma_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def library_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile ``gma_oracle.c`` with gcc (-O2, OpenMP, strict IEEE: no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
               "-Wextra", "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        d = ctypes.c_double
        lib.gma_oracle_log_joint.argtypes = [dp, i, i, dp, dp, dp, i, d, dp]
        lib.gma_oracle_log_joint.restype = i
        lib.gma_oracle_responsibilities.argtypes = [dp, i, i, dp, dp, dp, i, d, dp]
        lib.gma_oracle_responsibilities.restype = i
        lib.gma_oracle_forward.argtypes = [dp, dp, dp, dp, dp, dp, i, i, i, i, i, i, i, d, d,
                                           dp, dp, dp]
        lib.gma_oracle_forward.restype = i
        lib.gma_oracle_forward_cross.argtypes = [dp, dp, dp, dp, dp, dp, i, i, i, i, i, i, i, d, d,
                                                 dp, dp, dp]
        lib.gma_oracle_forward_cross.restype = i
        lib.gma_oracle_memory.argtypes = [dp, dp, dp, dp, dp, i, i, i, i, i, i, d, dp]
        lib.gma_oracle_memory.restype = i
        lib.gma_oracle_decode_step.argtypes = [dp, dp, dp, dp, dp, dp, i, i, i, i, i, d, d, dp, dp]
        lib.gma_oracle_decode_step.restype = i
        ip = ctypes.POINTER(ctypes.c_int)
        lp = ctypes.POINTER(ctypes.c_longlong)
        lib.gma_oracle_resp_stats.argtypes = [dp, dp, dp, dp, i, i, i, i, i, d, ip, lp, dp, ip, dp]
        lib.gma_oracle_resp_stats.restype = ctypes.c_int
        lib.gma_oracle_backward.argtypes = [dp, dp, dp, dp, dp, dp, dp, i, i, i, i, i, i, i, d, d,
                                            dp, dp, dp, dp, dp, dp]
        lib.gma_oracle_backward.restype = ctypes.c_int
        lib.gma_oracle_num_threads.argtypes = []
        lib.gma_oracle_num_threads.restype = i
        _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor (CPU)
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    return int(_load().gma_oracle_num_threads())


def log_joint(x, mu, var_raw, prior_logits, var_floor: float) -> np.ndarray:
    """log pi_k + log N(x_i; mu_k, diag var_k) for rows x [N, d] of one head -> [N, K]."""
    x, mu, vr, p = _f64(x), _f64(mu), _f64(var_raw), _f64(prior_logits)
    N, d = x.shape
    K = mu.shape[0]
    out = np.empty((N, K), dtype=np.float64)
    st = _load().gma_oracle_log_joint(_ptr(x), N, d, _ptr(mu), _ptr(vr), _ptr(p), K,
                                      float(var_floor), _ptr(out))
    if st != 0:
        raise RuntimeError(f"gma_oracle_log_joint failed: {st}")
    return out


def responsibilities(x, mu, var_raw, prior_logits, var_floor: float) -> np.ndarray:
    """GMM posterior p(z=k | x_i) for rows x [N, d] of one head -> [N, K]."""
    x, mu, vr, p = _f64(x), _f64(mu), _f64(var_raw), _f64(prior_logits)
    N, d = x.shape
    K = mu.shape[0]
    out = np.empty((N, K), dtype=np.float64)
    st = _load().gma_oracle_responsibilities(_ptr(x), N, d, _ptr(mu), _ptr(vr), _ptr(p), K,
                                             float(var_floor), _ptr(out))
    if st != 0:
        raise RuntimeError(f"gma_oracle_responsibilities failed: {st}")
    return out


def forward(qr, kr, v, mu, var_raw, prior_logits, causal: bool, eps: float,
            var_floor: float, return_gamma: bool = False
            ) -> np.ndarray | Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """fp64 GMA forward.  qr, kr [B,H,N,d_r]; v [B,H,N,d_v]; mu, var_raw [H,K,d_r];
    prior_logits [H,K].  Returns out [B,H,N,d_v] (and Gamma_Q, Gamma_K [B,H,N,K])."""
    qr, kr, v = _f64(qr), _f64(kr), _f64(v)
    mu, vr, p = _f64(mu), _f64(var_raw), _f64(prior_logits)
    B, H, N, d_r = qr.shape
    d_v = v.shape[-1]
    K = mu.shape[1]
    if kr.shape != qr.shape or v.shape[:3] != qr.shape[:3]:
        raise ValueError("shape mismatch")
    if mu.shape != (H, K, d_r) or vr.shape != (H, K, d_r) or p.shape != (H, K):
        raise ValueError("parameter shape mismatch")
    out = np.empty((B, H, N, d_v), dtype=np.float64)
    gq = np.empty((B, H, N, K), dtype=np.float64) if return_gamma else None
    gk = np.empty((B, H, N, K), dtype=np.float64) if return_gamma else None
    st = _load().gma_oracle_forward(_ptr(qr), _ptr(kr), _ptr(v), _ptr(mu), _ptr(vr), _ptr(p),
                                    B, H, N, d_r, d_v, K, 1 if causal else 0, float(eps),
                                    float(var_floor), _ptr(out), _ptr(gq), _ptr(gk))
    if st != 0:
        raise RuntimeError(f"gma_oracle_forward failed: {st}")
    if return_gamma:
        return out, gq, gk
    return out


def forward_cross(qr, kr, v, mu, var_raw, prior_logits, eps: float, var_floor: float,
                  return_gamma: bool = False):
    """fp64 cross variant (bidirectional).  qr [B,H,Nq,d_r]; kr [B,H,Nk,d_r]; v [B,H,Nk,d_v];
    mu, var_raw [H,K,d_r]; prior_logits [H,K].  Returns out [B,H,Nq,d_v] (and Gamma_Q
    [B,H,Nq,K], Gamma_K [B,H,Nk,K])."""
    qr, kr, v = _f64(qr), _f64(kr), _f64(v)
    mu, vr, p = _f64(mu), _f64(var_raw), _f64(prior_logits)
    B, H, Nq, d_r = qr.shape
    Nk = kr.shape[2]
    d_v = v.shape[-1]
    K = mu.shape[1]
    if kr.shape != (B, H, Nk, d_r) or v.shape[:3] != (B, H, Nk):
        raise ValueError("shape mismatch")
    if mu.shape != (H, K, d_r) or vr.shape != (H, K, d_r) or p.shape != (H, K):
        raise ValueError("parameter shape mismatch")
    out = np.empty((B, H, Nq, d_v), dtype=np.float64)
    gq = np.empty((B, H, Nq, K), dtype=np.float64) if return_gamma else None
    gk = np.empty((B, H, Nk, K), dtype=np.float64) if return_gamma else None
    st = _load().gma_oracle_forward_cross(_ptr(qr), _ptr(kr), _ptr(v), _ptr(mu), _ptr(vr), _ptr(p),
                                          B, H, Nq, Nk, d_r, d_v, K, float(eps), float(var_floor),
                                          _ptr(out), _ptr(gq), _ptr(gk))
    if st != 0:
        raise RuntimeError(f"gma_oracle_forward_cross failed: {st}")
    if return_gamma:
        return out, gq, gk
    return out


def memory(kr, v, mu, var_raw, prior_logits, var_floor: float) -> np.ndarray:
    """Causal memory [S | z] of the N positions of every (b, h): kr [B,H,N,d_r], v [B,H,N,d_v]
    -> state [B,H,K,d_v+1] (row k: S[k, :d_v], z[k])."""
    kr, v = _f64(kr), _f64(v)
    mu, vr, p = _f64(mu), _f64(var_raw), _f64(prior_logits)
    B, H, N, d_r = kr.shape
    d_v = v.shape[-1]
    K = mu.shape[1]
    state = np.empty((B, H, K, d_v + 1), dtype=np.float64)
    st = _load().gma_oracle_memory(_ptr(kr), _ptr(v), _ptr(mu), _ptr(vr), _ptr(p), B, H, N, d_r, d_v, K,
                                   float(var_floor), _ptr(state))
    if st != 0:
        raise RuntimeError(f"gma_oracle_memory failed: {st}")
    return state


def decode_step(qr, kr, v, mu, var_raw, prior_logits, state: np.ndarray, eps: float,
                var_floor: float) -> np.ndarray:
    """One causal decode step: qr, kr [B,H,d_r], v [B,H,d_v]; ``state`` [B,H,K,d_v+1] float64
    (C-contiguous) is updated in place; returns out [B,H,d_v]."""
    qr, kr, v = _f64(qr), _f64(kr), _f64(v)
    mu, vr, p = _f64(mu), _f64(var_raw), _f64(prior_logits)
    B, H, d_r = qr.shape
    d_v = v.shape[-1]
    K = mu.shape[1]
    if state.dtype != np.float64 or not state.flags.c_contiguous or state.shape != (B, H, K, d_v + 1):
        raise ValueError("state must be a C-contiguous float64 array [B,H,K,d_v+1]")
    out = np.empty((B, H, d_v), dtype=np.float64)
    st = _load().gma_oracle_decode_step(_ptr(qr), _ptr(kr), _ptr(v), _ptr(mu), _ptr(vr), _ptr(p), B, H, d_r,
                                        d_v, K, float(eps), float(var_floor), _ptr(state), _ptr(out))
    if st != 0:
        raise RuntimeError(f"gma_oracle_decode_step failed: {st}")
    return out


def resp_stats(x, mu, var_raw, prior_logits, var_floor: float) -> dict:
    """Responsibility statistics of the routing rows x [B,H,N,d_r] per head, pooled over the
    batch and the positions: ``hard`` int32 [B,H,N] (argmax, lowest index on ties),
    ``counts`` int64 [H,K], ``usage`` float64 [H,K] (sum of gamma), ``used`` int32 [H],
    ``entropy`` float64 [H] (hard-usage entropy over ln K)."""
    lib = _load()
    x, mu, vr, p = (_f64(a) for a in (x, mu, var_raw, prior_logits))
    B, H, N, d_r = x.shape
    K = mu.shape[1]
    hard = np.zeros((B, H, N), dtype=np.int32)
    counts = np.zeros((H, K), dtype=np.int64)
    usage = np.zeros((H, K), dtype=np.float64)
    used = np.zeros(H, dtype=np.int32)
    entropy = np.zeros(H, dtype=np.float64)
    ip = ctypes.POINTER(ctypes.c_int)
    st = lib.gma_oracle_resp_stats(_ptr(x), _ptr(mu), _ptr(vr), _ptr(p), B, H, N, d_r, K, float(var_floor),
                                   hard.ctypes.data_as(ip), counts.ctypes.data_as(ctypes.POINTER(ctypes.c_longlong)),
                                   _ptr(usage), used.ctypes.data_as(ip), _ptr(entropy))
    if st != 0:
        raise RuntimeError(f"oracle resp_stats failed: {st}")
    return {"hard": hard, "counts": counts, "usage": usage, "used": used, "entropy": entropy}


def backward(qr, kr, v, mu, var_raw, prior_logits, dout, causal: bool, eps: float, var_floor: float) -> dict:
    """Gradients of L = sum(dout * O) for the forward mixer: ``dqr``, ``dkr`` [B,H,N,d_r],
    ``dv`` [B,H,N,d_v], ``dmu``, ``dvar_raw`` [H,K,d_r], ``dprior`` [H,K] (float64)."""
    lib = _load()
    qr, kr, v, mu, vr, p, do = (_f64(a) for a in (qr, kr, v, mu, var_raw, prior_logits, dout))
    B, H, N, d_r = qr.shape
    d_v = v.shape[-1]
    K = mu.shape[1]
    out = {"dqr": np.zeros_like(qr), "dkr": np.zeros_like(kr), "dv": np.zeros_like(v), "dmu": np.zeros_like(mu),
           "dvar_raw": np.zeros_like(vr), "dprior": np.zeros_like(p)}
    st = lib.gma_oracle_backward(_ptr(qr), _ptr(kr), _ptr(v), _ptr(mu), _ptr(vr), _ptr(p), _ptr(do), B, H, N, d_r,
                                 d_v, K, 1 if causal else 0, float(eps), float(var_floor), _ptr(out["dqr"]),
                                 _ptr(out["dkr"]), _ptr(out["dv"]), _ptr(out["dmu"]), _ptr(out["dvar_raw"]),
                                 _ptr(out["dprior"]))
    if st != 0:
        raise RuntimeError(f"oracle backward failed: {st}")
    return out
