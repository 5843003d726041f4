"""Error metrics used by every parity check (GPU vs oracle).

Gate metric: the per-token (row) normwise relative error,
    max_{b,h,i} ||O_i - R_i||_inf / max(||R_i||_inf, 1e-3 * ||R_{b,h}||_inf),
floored per head so rows whose reference is tiny (eps-dominated or underflowed)
do not turn rounding noise into a huge ratio.  Outputs are convex-like
combinations of value rows and cross zero, so an elementwise relative error is
ill-posed; the row-normwise form is the plainest reading of "max relative error".
Also reported: the tensor-normwise ||O - R||_inf / ||R||_inf.
"""
import numpy as np

FP32_TOL = 1e-5
BF16_TOL = 2e-2


def _np(x):
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def rowrel(out, ref) -> float:
    o, r = _np(out), _np(ref)
    assert o.shape == r.shape, (o.shape, r.shape)
    if o.size == 0:
        return 0.0
    err = np.abs(o - r).max(axis=-1)
    rmax = np.abs(r).max(axis=-1)
    head = np.abs(r).max(axis=(-1, -2), keepdims=True)[..., 0]
    denom = np.maximum(rmax, 1e-3 * head)
    denom = np.where(denom > 0, denom, np.finfo(np.float64).tiny)
    return float((err / denom).max())


def globalrel(out, ref) -> float:
    o, r = _np(out), _np(ref)
    if o.size == 0:
        return 0.0
    return float(np.abs(o - r).max() / max(np.abs(r).max(), np.finfo(np.float64).tiny))


def tol_for(dtype: str) -> float:
    return FP32_TOL if dtype == "f32" else BF16_TOL


# Responsibilities of the matrix-core path (bf16 inputs): the logits come from the five-pass
# split contraction in fp32, so each gamma carries the logit error as a relative error:
# log2(g_k / r_k) = dl_k - log2(sum_j r_j 2^dl_j), at most 2 max_k |dl_k| (log2 units).
# The check takes entries whose reference is at least GAMMA_FLOOR (below it the fp32
# rounding of tiny values, not the logits, dominates; those entries are held to an
# absolute bound instead).  The bound on |log2(g/r)| is measured against what the split
# must deliver: a dropped hi/lo pass or a single bf16 operand gives logit errors of
# 0.1 to several units, far above it.
GAMMA_FLOOR = 1e-3
GAMMA_LOG2_TOL_BF16 = 2e-2
GAMMA_ABS_TOL_BF16 = 2e-5


def gamma_errors(g, ref):
    """(max |log2(g / ref)| over ref >= GAMMA_FLOOR, max |g - ref| over ref < GAMMA_FLOOR)."""
    gg, r = _np(g), _np(ref)
    assert gg.shape == r.shape, (gg.shape, r.shape)
    big = r >= GAMMA_FLOOR
    lr = 0.0
    if big.any():
        with np.errstate(divide="ignore"):
            lr = float(np.abs(np.log2(np.maximum(gg[big], 1e-300) / r[big])).max())
    ab = float(np.abs(gg[~big] - r[~big]).max()) if (~big).any() else 0.0
    return lr, ab
