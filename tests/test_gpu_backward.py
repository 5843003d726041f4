"""GPU parity of the backward (gma_backward) against the fp64 oracle's chain rule.

Every gradient is compared row by row (the last dimension is the row: d_r or d_v for the
input-row gradients, the routing dims for dmu and dvar_raw, the components for dprior):
row-normwise relative error <= 1e-5 for float32 inputs and <= 2e-2 for bf16 inputs (whose
dqr, dkr, dv are rounded to bf16), the same gate as the forward.
"""
import sys

import numpy as np
import pytest

import oracle
from tests import metrics

torch = pytest.importorskip("torch")
gma = pytest.importorskip("gaussian_mixture_sequence_resp_amd")
from gaussian_mixture_sequence_resp_amd.inputs import WORKLOADS, make_inputs  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NAMES = ("dqr", "dkr", "dv", "dmu", "dvar_raw", "dprior")


def _say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def _dout(w, seed):
    g = torch.Generator().manual_seed(seed)
    d = torch.randn(w.B, w.H, w.N, w.d_v, generator=g)
    return d.to(torch.bfloat16) if w.dtype == "bf16" else d


def _compare(got, ref, tol):
    errs = {}
    for n in NAMES:
        a = got[n].float().cpu().numpy().astype(np.float64)
        r = ref[n]
        if n == "dprior":
            a, r = a[None, None], r[None, None]          # rows = components of a head
        elif n in ("dmu", "dvar_raw"):
            a, r = a[None], r[None]                      # rows = (h, k)
        assert np.all(np.isfinite(a)), n
        errs[n] = metrics.rowrel(a, r) if r.size else 0.0
    bad = {n: e for n, e in errs.items() if e > tol}
    assert not bad, (bad, errs)
    return errs


SHAPES = [
    # (B, H, N, d_r, d_v, K)
    (2, 3, 37, 16, 8, 12), (1, 2, 130, 64, 64, 128), (2, 2, 65, 24, 40, 33), (1, 1, 1, 8, 8, 1),
    (1, 2, 50, 5, 7, 7), (1, 1, 300, 64, 64, 256), (1, 1, 40, 128, 128, 256),
    # enough (b, h) x positions that each head's rows are cut into segments of several
    # 16-position chunks (32 and 64 rows per segment, the last one ragged)
    (4, 4, 4096, 16, 16, 32), (4, 8, 4000, 16, 24, 20),
    # state widths at the 32-column tile edges (d_v + 1 = 96 and 32), K padded within a tile
    (1, 2, 100, 32, 95, 96), (2, 1, 70, 8, 31, 64),
    # causal bf16 chunk walk on the matrix cores: d_v = 32 and 64, K within a tile (ragged,
    # not a multiple of 4), segments and their last chunks ragged
    (4, 4, 1000, 16, 32, 64), (2, 4, 777, 32, 64, 99),
    # eight component tiles (two waves per segment, each half the components): K not a multiple
    # of 4 with the second wave's components mostly padding, and d_v = 32
    (2, 2, 333, 64, 64, 131), (1, 3, 250, 32, 32, 200),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,H,N,dr,dv,K", SHAPES)
def test_backward_matches_oracle(B, H, N, dr, dv, K, dtype, causal):
    w = WORKLOADS[3].with_(B=B, H=H, N=N, d_r=dr, d_v=dv, K=K, dtype=dtype, causal=causal,
                           seed=131 + N + K + dr + causal)
    inp = make_inputs(w)
    dout = _dout(w, w.seed + 7)
    _say("backward", dtype, "causal" if causal else "bidir", dict(B=B, H=H, N=N, dr=dr, dv=dv, K=K, seed=w.seed))
    d = {k: x.to(DEV) for k, x in inp.items()}
    got = gma.backward(d["qr"], d["kr"], d["v"], d["mu"], d["var_raw"], d["prior_logits"], dout.to(DEV), causal,
                       eps=w.eps, var_floor=w.var_floor)
    torch.cuda.synchronize()
    ref = oracle.backward(inp["qr"], inp["kr"], inp["v"], inp["mu"], inp["var_raw"], inp["prior_logits"], dout,
                          causal, w.eps, w.var_floor)
    errs = _compare(got, ref, metrics.tol_for(dtype))
    _say("backward errors", {n: f"{e:.2e}" for n, e in errs.items()})


def test_backward_deterministic_and_empty():
    w = WORKLOADS[3].with_(B=2, H=2, N=90, K=40, d_r=16, d_v=16, seed=141)
    inp = make_inputs(w)
    d = {k: x.to(DEV) for k, x in inp.items()}
    dout = _dout(w, 142).to(DEV)
    for causal in (False, True):
        g1 = gma.backward(d["qr"], d["kr"], d["v"], d["mu"], d["var_raw"], d["prior_logits"], dout, causal)
        g2 = gma.backward(d["qr"], d["kr"], d["v"], d["mu"], d["var_raw"], d["prior_logits"], dout, causal)
        torch.cuda.synchronize()
        for n in NAMES:
            assert torch.equal(g1[n], g2[n]), n
    # no positions: zero parameter gradients
    w0 = w.with_(N=0)
    inp0 = make_inputs(w0)
    d0 = {k: x.to(DEV) for k, x in inp0.items()}
    g0 = gma.backward(d0["qr"], d0["kr"], d0["v"], d0["mu"], d0["var_raw"], d0["prior_logits"],
                      torch.empty(2, 2, 0, 16, dtype=torch.bfloat16, device=DEV), True)
    torch.cuda.synchronize()
    for n in ("dmu", "dvar_raw", "dprior"):
        assert int(torch.count_nonzero(g0[n])) == 0, n


@pytest.mark.parametrize("cfg", [2, 3])
def test_backward_full_size_sampled_heads(cfg):
    """The backward at the benchmark's full sizes (the bidirectional K=128 and causal LM
    workloads, the launch configuration the benchmark times), every gradient of two heads
    (0 and H-1, all batch elements) against the oracle run on those heads alone: heads are
    independent, so each is an H = 1 problem with that head's parameters."""
    w = WORKLOADS[cfg]
    inp = make_inputs(w)
    dout = _dout(w, w.seed + 7)
    _say("backward full size", w.name, dict(B=w.B, H=w.H, N=w.N, K=w.K))
    d = {k: x.to(DEV) for k, x in inp.items()}
    got = gma.backward(d["qr"], d["kr"], d["v"], d["mu"], d["var_raw"], d["prior_logits"], dout.to(DEV), w.causal,
                       eps=w.eps, var_floor=w.var_floor)
    torch.cuda.synchronize()
    for h in (0, w.H - 1):
        sub = {k: (x[:, h:h + 1].contiguous() if k in ("qr", "kr", "v") else x[h:h + 1].contiguous())
               for k, x in inp.items()}
        ref = oracle.backward(sub["qr"], sub["kr"], sub["v"], sub["mu"], sub["var_raw"], sub["prior_logits"],
                              dout[:, h:h + 1].contiguous(), w.causal, w.eps, w.var_floor)
        mine = {n: (got[n][:, h:h + 1] if n in ("dqr", "dkr", "dv") else got[n][h:h + 1]) for n in NAMES}
        errs = _compare(mine, ref, metrics.tol_for(w.dtype))
        _say("backward full size head", h, {n: f"{e:.2e}" for n, e in errs.items()})
