"""GPU parity of the cross variant (queries and keys of different lengths) against the
fp64 oracle, through the C ABI (gma_forward_cross).

Reading (German page, closing paragraph: cross-attention as future work): the
bidirectional write over the N_k key rows and the read by the N_q query rows.  Gate as
for the self-mixing forward: row-normwise relative error <= 1e-5 (float32 inputs),
<= 2e-2 (bf16 inputs).
"""
import sys

import numpy as np
import pytest

import oracle
from tests import metrics

torch = pytest.importorskip("torch")
gma = pytest.importorskip("gaussian_mixture_sequence_resp_amd")
from gaussian_mixture_sequence_resp_amd.inputs import WORKLOADS, Workload, make_inputs  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def _supported(w: Workload, algo: str) -> bool:
    if algo == "simt":
        return True
    if w.dtype != "bf16":
        return False
    desc = gma.make_desc(w.B, w.H, w.N, w.d_r, w.d_v, w.K, w.dtype, w.var_floor, algo)
    return gma.workspace_size_cross(desc, w.Nk) > 0


def run_cross(inp, w: Workload, algo="auto", want_gamma=False):
    d = {k: v.to(DEV) for k, v in inp.items()}
    gamma = None
    if want_gamma:
        gamma = torch.empty(w.B * w.H * (w.N + w.Nk) * w.K, dtype=torch.float32, device=DEV)
    out = gma.forward_cross(d["qr"], d["kr"], d["v"], d["mu"], d["var_raw"], d["prior_logits"],
                            eps=w.eps, var_floor=w.var_floor, gamma_out=gamma, algo=algo)
    torch.cuda.synchronize()
    return out.cpu(), (gamma.cpu() if gamma is not None else None)


def oracle_cross(inp, w: Workload, heads=None, want_gamma=False):
    if heads is None:
        return oracle.forward_cross(inp["qr"], inp["kr"], inp["v"], inp["mu"], inp["var_raw"],
                                    inp["prior_logits"], w.eps, w.var_floor, return_gamma=want_gamma)
    outs = []
    for b, h in heads:
        sl = slice(b, b + 1), slice(h, h + 1)
        outs.append(oracle.forward_cross(inp["qr"][sl], inp["kr"][sl], inp["v"][sl], inp["mu"][h:h + 1],
                                         inp["var_raw"][h:h + 1], inp["prior_logits"][h:h + 1], w.eps,
                                         w.var_floor)[0, 0])
    return outs


CROSS = [
    # (N_q, N_k, K, d_r, d_v)
    (1, 1, 1, 8, 8), (17, 300, 64, 64, 64), (300, 17, 128, 64, 64), (1000, 4096, 128, 64, 64),
    (513, 129, 33, 104, 72), (200, 5000, 256, 24, 40), (257, 777, 5, 3, 7), (2048, 31, 256, 128, 128),
]


@pytest.mark.parametrize("algo", ["simt", "mfma"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Nq,Nk,K,dr,dv", CROSS)
def test_cross_shapes(Nq, Nk, K, dr, dv, dtype, algo):
    w = WORKLOADS[2].with_(B=2, H=2, N=Nq, N_k=Nk, K=K, d_r=dr, d_v=dv, dtype=dtype, seed=31 + Nq + Nk)
    if not _supported(w, algo):
        pytest.skip(f"{algo} does not cover {dtype} {w}")
    inp = make_inputs(w)
    _say("cross", algo, dtype, dict(Nq=Nq, Nk=Nk, K=K, dr=dr, dv=dv, seed=w.seed))
    out, _ = run_cross(inp, w, algo)
    ref = oracle_cross(inp, w)
    assert out.shape == (2, 2, Nq, dv)
    assert np.all(np.isfinite(out.float().numpy()))
    err = metrics.rowrel(out, ref)
    assert err <= metrics.tol_for(dtype), (err, metrics.globalrel(out, ref))


@pytest.mark.parametrize("algo", ["simt", "mfma"])
def test_cross_empty_memory_is_zero(algo):
    w = WORKLOADS[2].with_(B=2, H=2, N=300, N_k=0, K=64, seed=5)
    inp = make_inputs(w)
    _say("cross empty memory", algo)
    out, _ = run_cross(inp, w, algo)
    assert torch.count_nonzero(out) == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cross_gamma_out_matches_oracle(dtype):
    w = WORKLOADS[2].with_(B=1, H=3, N=200, N_k=333, K=64, dtype=dtype, seed=98)
    inp = make_inputs(w)
    _say("cross gamma_out", dtype)
    _, gam = run_cross(inp, w, "auto", want_gamma=True)
    _, gq, gk = oracle_cross(inp, w, want_gamma=True)
    nq = w.B * w.H * w.N * w.K
    np.testing.assert_allclose(gam[:nq].numpy().reshape(gq.shape), gq, atol=1e-5)
    np.testing.assert_allclose(gam[nq:].numpy().reshape(gk.shape), gk, atol=1e-5)


@pytest.mark.parametrize("algo", ["simt", "mfma"])
def test_cross_with_the_same_rows_is_self_mixing_bitwise(algo):
    w = WORKLOADS[2].with_(B=2, H=2, N=1111, seed=77)
    inp = make_inputs(w)
    _say("cross == self", algo)
    d = {k: v.to(DEV) for k, v in inp.items()}
    o1 = gma.forward(d["qr"], d["kr"], d["v"], d["mu"], d["var_raw"], d["prior_logits"], causal=False,
                     eps=w.eps, var_floor=w.var_floor, algo=algo)
    o2 = gma.forward_cross(d["qr"], d["kr"], d["v"], d["mu"], d["var_raw"], d["prior_logits"], eps=w.eps,
                           var_floor=w.var_floor, algo=algo)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_cross_full_size_sampled():
    # the benchmark's cross shape: 1024 queries read a memory of 16384 keys
    w = WORKLOADS[2].with_(N=1024, N_k=16384, seed=1006)
    inp = make_inputs(w)
    _say("cross full size", w)
    out, _ = run_cross(inp, w)
    heads = [(0, 0), (w.B - 1, w.H - 1), (w.B // 2, w.H // 2)]
    refs = oracle_cross(inp, w, heads=heads)
    err = max(metrics.rowrel(out[b, h][None, None], r[None, None]) for (b, h), r in zip(heads, refs))
    _say("cross full size rowrel", err)
    assert err <= metrics.tol_for(w.dtype), err
