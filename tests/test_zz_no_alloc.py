"""gma_forward_noalloc (the library's static scratch, no workspace argument) against
gma_forward (caller's workspace) through the C ABI: two calls in a row on one stream, the
second with a smaller input, each bitwise equal to gma_forward on the same inputs (same
kernels; the only difference is where the scratch lives), and both within the oracle's bf16
gate.  Bidirectional and causal, matrix-core and SIMT families."""
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


def _pair(w, algo):
    inp = make_inputs(w)
    d = {k: v.to(DEV) for k, v in inp.items()}
    ref_ws = gma.forward(d["qr"], d["kr"], d["v"], d["mu"], d["var_raw"], d["prior_logits"], causal=w.causal,
                         eps=w.eps, var_floor=w.var_floor, algo=algo)
    out = torch.empty_like(ref_ws)
    gma.forward_noalloc(d["qr"], d["kr"], d["v"], d["mu"], d["var_raw"], d["prior_logits"], out,
                        causal=w.causal, eps=w.eps, var_floor=w.var_floor, algo=algo)
    torch.cuda.synchronize()
    return inp, ref_ws.cpu(), out.cpu()


@pytest.mark.parametrize("algo", ["auto", "simt"])
@pytest.mark.parametrize("cfg", [2, 3])
def test_noalloc_matches_forward_two_calls(cfg, algo):
    big = WORKLOADS[cfg].with_(B=2, H=4, N=2000, seed=31 + cfg)
    small = WORKLOADS[cfg].with_(B=1, H=3, N=333, seed=41 + cfg)
    for w in (big, small):
        print("[gpu-case] noalloc", algo, w, file=sys.stderr, flush=True)
        inp, ref_ws, out = _pair(w, algo)
        assert torch.equal(out, ref_ws)
        ref = oracle.forward(inp["qr"], inp["kr"], inp["v"], inp["mu"], inp["var_raw"], inp["prior_logits"],
                             w.causal, w.eps, w.var_floor)
        assert np.all(np.isfinite(out.float().numpy()))
        assert metrics.rowrel(out, ref) <= metrics.tol_for(w.dtype)


def test_noalloc_rejects_beyond_scratch():
    w = WORKLOADS[2].with_(B=64, H=8, N=8192)
    d = {"qr": torch.empty((w.B, w.H, w.N, w.d_r), dtype=torch.bfloat16, device=DEV)}
    d["kr"] = torch.empty_like(d["qr"])
    d["v"] = torch.empty((w.B, w.H, w.N, w.d_v), dtype=torch.bfloat16, device=DEV)
    p = {k: torch.zeros(s, device=DEV) for k, s in (("mu", (w.H, w.K, w.d_r)), ("var_raw", (w.H, w.K, w.d_r)),
                                                    ("prior_logits", (w.H, w.K)))}
    out = torch.empty_like(d["v"])
    with pytest.raises(gma.GMAError) as ei:
        gma.forward_noalloc(d["qr"], d["kr"], d["v"], p["mu"], p["var_raw"], p["prior_logits"], out, algo="simt")
    assert ei.value.code == -9
