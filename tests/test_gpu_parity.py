"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Gate (row-normwise relative error, see tests/metrics.py): <= 1e-5 for float32
inputs, <= 2e-2 for bf16 inputs with fp32 accumulation.  Every case prints its name,
shape and seed before the GPU call so a failure is attributable.
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


def _algo_supported(w: Workload, algo: str) -> bool:
    if algo == "simt":
        return True
    if w.dtype != "bf16":
        return False
    desc = gma.make_desc(w.B, w.H, w.N, w.d_r, w.d_v, w.K, w.dtype, w.var_floor, algo)
    return gma.workspace_size(desc, w.causal) > 0


def run_gpu(inp, w: Workload, algo="auto", want_gamma=False):
    d = {k: v.to(DEV) for k, v in inp.items()}
    gamma = None
    if want_gamma:
        gamma = torch.empty((2, w.B, w.H, w.N, w.K), dtype=torch.float32, device=DEV)
    out = gma.forward(d["qr"], d["kr"], d["v"], d["mu"], d["var_raw"], d["prior_logits"],
                      causal=w.causal, eps=w.eps, var_floor=w.var_floor, gamma_out=gamma, algo=algo)
    torch.cuda.synchronize()
    return out.cpu(), (gamma.cpu() if gamma is not None else None)


def run_oracle(inp, w: Workload, heads=None, want_gamma=False):
    """fp64 oracle on all (b, h) slices, or only on the listed ones."""
    if heads is None:
        return oracle.forward(inp["qr"], inp["kr"], inp["v"], inp["mu"], inp["var_raw"],
                              inp["prior_logits"], w.causal, w.eps, w.var_floor,
                              return_gamma=want_gamma)
    outs = []
    for b, h in heads:
        sl = slice(b, b + 1), slice(h, h + 1)
        outs.append(oracle.forward(inp["qr"][sl], inp["kr"][sl], inp["v"][sl],
                                   inp["mu"][h:h + 1], inp["var_raw"][h:h + 1],
                                   inp["prior_logits"][h:h + 1], w.causal, w.eps, w.var_floor)[0, 0])
    return outs


SMALL = [
    # (N, K, d_r, d_v, causal)
    (1, 1, 1, 1, False), (1, 3, 5, 7, True), (7, 8, 16, 16, False), (33, 5, 3, 9, True),
    (100, 64, 64, 64, False), (100, 64, 64, 64, True), (257, 128, 64, 64, False),
    (257, 256, 64, 64, True), (300, 17, 40, 24, False), (129, 256, 128, 128, True),
    (512, 128, 64, 64, True), (1000, 33, 100, 128, False),
    # ragged within the padded tiles on the matrix-core path (dims multiples of 8)
    (1000, 33, 104, 72, False), (777, 200, 24, 40, True),
    # small tiles (K <= 64, d <= 64): the write at two workgroups per CU over 8 splits, a
    # ragged last split, then the split reduce
    (1000, 40, 48, 56, False),
    # 256 padded components of 128 padded routing dims, causal: the component-parallel
    # responsibilities (one wave's 32 components all padding), four parts, a ragged tail
    (1000, 200, 120, 64, True),
]


@pytest.mark.parametrize("algo", ["simt", "mfma"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,K,dr,dv,causal", SMALL)
def test_small_shapes(N, K, dr, dv, causal, dtype, algo):
    w = WORKLOADS[2].with_(B=2, H=2, N=N, K=K, d_r=dr, d_v=dv, causal=causal, dtype=dtype,
                           seed=7 + N + K)
    if not _algo_supported(w, algo):
        pytest.skip(f"{algo} does not cover {dtype} {w}")
    inp = make_inputs(w)
    _say("small", algo, dtype, dict(N=N, K=K, dr=dr, dv=dv, causal=causal, seed=w.seed))
    out, _ = run_gpu(inp, w, algo)
    ref = run_oracle(inp, w)
    err = metrics.rowrel(out, ref)
    assert np.all(np.isfinite(out.float().numpy()))
    assert err <= metrics.tol_for(dtype), (err, metrics.globalrel(out, ref))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workloads_full_size(cfg):
    """Every workload at its full size, in the launch configuration the benchmark times
    (algo auto), against the oracle on every (b, h) slice."""
    w = WORKLOADS[cfg]
    inp = make_inputs(w)
    _say("workload", cfg, w)
    out, _ = run_gpu(inp, w, "auto")
    assert np.all(np.isfinite(out.float().numpy()))
    _say("workload", cfg, "oracle over all", w.B * w.H, "heads")
    ref = run_oracle(inp, w)
    per_head = [metrics.rowrel(out[b, h][None, None], ref[b, h][None, None])
                for b in range(w.B) for h in range(w.H)]
    err = max(per_head)
    _say("workload", cfg, "rowrel max", f"{err:.3e}", "median head", f"{float(np.median(per_head)):.3e}",
         "global", f"{metrics.globalrel(out, ref):.3e}")
    assert err <= metrics.tol_for(w.dtype), err


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_responsibilities_full_size(cfg):
    """The matrix-core responsibilities (gamma_out: the same five-pass split logits and
    softmax as the fused kernels) at each workload's full shape, both sides, every (b, h),
    against the oracle's fp64 posteriors: the logit precision of the split contraction."""
    w = WORKLOADS[cfg]
    inp = make_inputs(w)
    _say("responsibilities", cfg, w)
    _, gam = run_gpu(inp, w, "auto", want_gamma=True)
    worst_lr, worst_ab = 0.0, 0.0
    for b in range(w.B):  # one batch element at a time bounds the oracle's fp64 copies
        sl = slice(b, b + 1)
        _, gq, gk = oracle.forward(inp["qr"][sl], inp["kr"][sl], inp["v"][sl], inp["mu"], inp["var_raw"],
                                   inp["prior_logits"], w.causal, w.eps, w.var_floor, return_gamma=True)
        for side, ref in ((0, gq), (1, gk)):
            lr, ab = metrics.gamma_errors(gam[side, b], ref[0])
            worst_lr, worst_ab = max(worst_lr, lr), max(worst_ab, ab)
        assert np.allclose(gam[:, b].sum(-1).numpy(), 1.0, atol=1e-5)
    _say("responsibilities", cfg, "max |log2(g/ref)|", f"{worst_lr:.3e}", "max abs (small)", f"{worst_ab:.3e}")
    assert worst_lr <= metrics.GAMMA_LOG2_TOL_BF16, worst_lr
    assert worst_ab <= metrics.GAMMA_ABS_TOL_BF16, worst_ab


def test_golden_fixture():
    import json
    import os
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_gma.json")))
    inp = {k: np.asarray(v) for k, v in fx["inputs"].items()}
    for dtype in ("f32", "bf16"):
        tdt = torch.float32 if dtype == "f32" else torch.bfloat16
        t = {k: torch.tensor(v, dtype=torch.float32) for k, v in inp.items()}
        for k in ("qr", "kr", "v"):
            t[k] = t[k].to(tdt)  # values are exact binary fractions: lossless in bf16
        B, H, N, dr = inp["qr"].shape
        for key, causal in (("bidirectional", False), ("causal", True)):
            w = Workload("golden", dtype, causal, B, H, N, dr, inp["v"].shape[-1], inp["mu"].shape[1],
                         seed=0, eps=fx["eps"], var_floor=fx["var_floor"])
            _say("golden", dtype, key)
            out, gam = run_gpu(t, w, "auto", want_gamma=True)
            ref = np.asarray(fx[key]["out"])
            assert metrics.rowrel(out, ref) <= metrics.tol_for(dtype)
            _assert_gamma(gam, np.stack([fx[key]["gamma_q"], fx[key]["gamma_k"]]), dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gamma_out_matches_oracle(dtype):
    w = WORKLOADS[2].with_(B=1, H=3, N=300, K=64, dtype=dtype, seed=99)
    inp = make_inputs(w)
    _say("gamma_out", dtype)
    _, gam = run_gpu(inp, w, "auto", want_gamma=True)
    _, gq, gk = run_oracle(inp, w, want_gamma=True)
    _assert_gamma(gam, np.stack([gq, gk]), dtype)
    np.testing.assert_allclose(gam.sum(-1).numpy(), 1.0, atol=1e-5)


def _assert_gamma(gam, ref, dtype):
    """float32 inputs: the SIMT responsibilities (double logits) to 1e-5 absolute; bf16
    inputs: the matrix-core responsibilities to the split contraction's logit precision."""
    if dtype == "f32":
        np.testing.assert_allclose(gam.numpy(), ref, atol=1e-5)
        return
    lr, ab = metrics.gamma_errors(gam, ref)
    assert lr <= metrics.GAMMA_LOG2_TOL_BF16 and ab <= metrics.GAMMA_ABS_TOL_BF16, (lr, ab)


@pytest.mark.parametrize("cfg", [3, 5])
def test_causal_outputs_ignore_future_bitwise(cfg):
    w = WORKLOADS[cfg].with_(B=1, H=2, N=1500)
    inp = make_inputs(w)
    cut = 777
    _say("causality", cfg, "cut", cut)
    out1, _ = run_gpu(inp, w)
    inp2 = {k: v.clone() for k, v in inp.items()}
    g = torch.Generator().manual_seed(5)
    for k in ("qr", "kr", "v"):
        x = inp2[k]
        x[:, :, cut + 1:] = (3 * torch.randn(x[:, :, cut + 1:].shape, generator=g)).to(x.dtype)
    out2, _ = run_gpu(inp2, w)
    assert torch.equal(out1[:, :, :cut + 1], out2[:, :, :cut + 1])
    assert not torch.equal(out1[:, :, cut + 1:], out2[:, :, cut + 1:])


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_deterministic_bitwise(cfg):
    w = WORKLOADS[cfg].with_(B=2, H=2, N=3000)
    inp = make_inputs(w)
    _say("determinism", cfg)
    out1, _ = run_gpu(inp, w)
    out2, _ = run_gpu(inp, w)
    assert torch.equal(out1, out2)
