"""GPU parity of the responsibility statistics (gma_resp_stats) against the fp64 oracle.

Hard assignments are an argmax decided in floating point: the kernel decides on its own
logits (fp32 on the matrix cores for bf16 inputs, double on the SIMT path), the oracle on
fp64 ones.  Rows whose two best components are separated by more than the kernel's logit
precision (DELTA, natural-log units) must agree exactly; for the others the kernel's choice
must be within DELTA of the best (a valid near-tie answer).  Counts must equal the histogram
of the kernel's own hard assignments exactly and differ from the oracle's by at most the
near-tie rows; used and entropy follow from the counts.  Soft usage: relative to the largest
entry, <= 1e-5 (float32 inputs), <= 2e-2 (bf16 inputs).
"""
import sys

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
gma = pytest.importorskip("gaussian_mixture_sequence_resp_amd")
from gaussian_mixture_sequence_resp_amd.inputs import WORKLOADS, make_inputs  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
# logit precision of the two paths, natural-log units.  Matrix cores: fp32 sums of exact bf16
# products; the dropped lo*lo split term is ~2^-18 of each |a x^2| term and fp32 accumulation
# adds ~2^-24 |l| per step, so with |l| <= ~450 and d_r <= 128 the error stays below ~5e-3
# (measured: 9e-5 at the causal-LM shape, 3 disagreeing rows of 262144).  SIMT: double.
DELTA = {"mfma": 1e-2, "simt": 1e-8}
USAGE_TOL = {"f32": 1e-5, "bf16": 2e-2}


def _say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def _check(inp, w, res, path):
    x = inp["kr"]
    ref = oracle.resp_stats(x, inp["mu"], inp["var_raw"], inp["prior_logits"], w.var_floor)
    lj = np.zeros((w.B, w.H, w.N, w.K))
    for b in range(w.B):
        for h in range(w.H):
            if w.N:
                lj[b, h] = oracle.log_joint(x[b, h], inp["mu"][h], inp["var_raw"][h], inp["prior_logits"][h],
                                            w.var_floor)
    H, K = w.H, w.K
    hard = res["hard"].cpu().numpy()
    counts = res["counts"].cpu().numpy()
    usage = res["usage"].cpu().numpy().astype(np.float64)
    used = res["used"].cpu().numpy()
    ent = res["entropy"].cpu().numpy().astype(np.float64)
    delta = DELTA[path]
    if w.N > 0:
        srt = np.sort(lj, axis=-1)
        margin = srt[..., -1] - srt[..., -2] if K > 1 else np.full(lj.shape[:-1], np.inf)
        clear = margin > delta
        assert ((hard >= 0) & (hard < K)).all()
        np.testing.assert_array_equal(hard[clear], ref["hard"][clear])
        chosen = np.take_along_axis(lj, hard[..., None].astype(np.int64), axis=-1)[..., 0]
        assert (chosen >= srt[..., -1] - delta).all()
        n_tie = int((~clear).sum())
    else:
        n_tie = 0
    # counts: exactly the histogram of the kernel's own assignments
    for h in range(H):
        own = np.bincount(hard[:, h].reshape(-1), minlength=K) if w.N > 0 else np.zeros(K, np.int64)
        np.testing.assert_array_equal(counts[h], own)
        assert used[h] == np.count_nonzero(own)
        rows = w.B * w.N
        p = own[own > 0] / rows if rows else np.zeros(0)
        ref_ent = float(-(p * np.log(p)).sum() / np.log(K)) if (K > 1 and rows) else 0.0
        assert abs(ent[h] - ref_ent) <= 1e-6, (h, ent[h], ref_ent)
    assert np.abs(counts - ref["counts"]).sum() <= 2 * n_tie
    if n_tie == 0:
        np.testing.assert_array_equal(used, ref["used"])
        np.testing.assert_allclose(ent, ref["entropy"], rtol=0, atol=1e-6)
    scale = max(float(np.abs(ref["usage"]).max()), 1e-30)
    err = float(np.abs(usage - ref["usage"]).max()) / scale
    assert err <= USAGE_TOL[w.dtype], err
    return n_tie


SHAPES = [
    # (B, H, N, d_r, K)
    (2, 3, 300, 64, 128), (2, 3, 300, 64, 256), (2, 2, 77, 24, 33), (1, 2, 50, 5, 7), (3, 1, 129, 16, 1),
    (1, 1, 1, 8, 16), (2, 2, 200, 128, 256),
]


def _path(dtype, algo, dr):
    return "mfma" if (dtype == "bf16" and algo != "simt" and dr % 8 == 0) else "simt"


@pytest.mark.parametrize("algo", ["auto", "simt"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,H,N,dr,K", SHAPES)
def test_stats_match_oracle(B, H, N, dr, K, dtype, algo):
    w = WORKLOADS[3].with_(B=B, H=H, N=N, d_r=dr, d_v=8, K=K, dtype=dtype, seed=81 + N + K + dr)
    inp = make_inputs(w)
    path = _path(dtype, algo, dr)
    _say("stats", dtype, algo, path, dict(B=B, H=H, N=N, dr=dr, K=K, seed=w.seed))
    d = {k: v.to(DEV) for k, v in inp.items()}
    res = gma.resp_stats(d["kr"], d["mu"], d["var_raw"], d["prior_logits"], var_floor=w.var_floor, algo=algo)
    torch.cuda.synchronize()
    _check(inp, w, res, path)


@pytest.mark.parametrize("algo", ["auto", "simt"])
def test_stats_empty_rows_and_no_hard_output(algo):
    w = WORKLOADS[3].with_(B=2, H=2, N=0, d_v=8, K=16, seed=91)
    inp = make_inputs(w)
    d = {k: v.to(DEV) for k, v in inp.items()}
    res = gma.resp_stats(d["kr"], d["mu"], d["var_raw"], d["prior_logits"], var_floor=w.var_floor, algo=algo)
    torch.cuda.synchronize()
    assert int(res["counts"].abs().sum()) == 0 and float(res["usage"].abs().sum()) == 0.0
    assert int(res["used"].sum()) == 0 and float(res["entropy"].abs().sum()) == 0.0
    # without the hard output: the same counts and usage as with it, bitwise
    w = WORKLOADS[3].with_(B=2, H=2, N=150, d_v=8, K=40, seed=92)
    inp = make_inputs(w)
    d = {k: v.to(DEV) for k, v in inp.items()}
    r1 = gma.resp_stats(d["kr"], d["mu"], d["var_raw"], d["prior_logits"], var_floor=w.var_floor, algo=algo)
    r2 = gma.resp_stats(d["kr"], d["mu"], d["var_raw"], d["prior_logits"], var_floor=w.var_floor, algo=algo,
                        with_hard=False)
    torch.cuda.synchronize()
    for k in ("counts", "usage", "used", "entropy"):
        assert torch.equal(r1[k], r2[k]), k


def test_stats_deterministic_and_full_size():
    # the causal-LM workload's shape (B=16, H=8, N=2048, K=256, d_r=64), key rows, matrix cores
    w = WORKLOADS[3]
    inp = make_inputs(w)
    _say("stats full size", w.name)
    d = {k: v.to(DEV) for k, v in inp.items()}
    r1 = gma.resp_stats(d["kr"], d["mu"], d["var_raw"], d["prior_logits"], var_floor=w.var_floor)
    r2 = gma.resp_stats(d["kr"], d["mu"], d["var_raw"], d["prior_logits"], var_floor=w.var_floor)
    torch.cuda.synchronize()
    for k in r1:
        assert torch.equal(r1[k], r2[k]), k
    n_tie = _check(inp, w, r1, "mfma")
    _say("stats full size near-tie rows", n_tie, "of", w.B * w.H * w.N)
