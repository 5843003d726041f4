"""GPU parity on hypothesis-drawn shapes: both kernel families (through the C ABI) against
the fp64 oracle on small random problems -- sequence lengths that are ragged against every
tile, components and dims on and off the matrix-core tile edges, both variants and dtypes.
The draw is derandomized (a fixed example database-free sequence), so a failure reproduces;
each example prints its shape and seed before its GPU call."""
import sys

import numpy as np
import pytest

import oracle
from tests import metrics

torch = pytest.importorskip("torch")
hyp = pytest.importorskip("hypothesis")
gma = pytest.importorskip("gaussian_mixture_sequence_resp_amd")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

from gaussian_mixture_sequence_resp_amd.inputs import WORKLOADS, make_inputs  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _dims(draw, mult8):
    if mult8:
        return 8 * draw(st.integers(1, 16))
    return draw(st.integers(1, 128))


@st.composite
def problems(draw):
    mult8 = draw(st.booleans())
    return dict(B=draw(st.integers(1, 2)), H=draw(st.integers(1, 3)),
                N=draw(st.one_of(st.integers(1, 40), st.integers(41, 700))),
                K=draw(st.one_of(st.integers(1, 40), st.integers(41, 256))),
                d_r=_dims(draw, mult8), d_v=_dims(draw, mult8), causal=draw(st.booleans()),
                dtype=draw(st.sampled_from(["f32", "bf16"])), seed=draw(st.integers(0, 10 ** 6)),
                var_floor=draw(st.sampled_from([1e-3, 1e-2])), mu_std=draw(st.sampled_from([1.0, 2.0])))


@settings(max_examples=40, deadline=None, derandomize=True, database=None,
          suppress_health_check=list(HealthCheck))
@given(p=problems())
def test_random_shapes_both_families(p):
    w = WORKLOADS[2].with_(B=p["B"], H=p["H"], N=p["N"], K=p["K"], d_r=p["d_r"], d_v=p["d_v"],
                           causal=p["causal"], dtype=p["dtype"], seed=p["seed"], var_floor=p["var_floor"],
                           mu_std=p["mu_std"])
    inp = make_inputs(w)
    ref = oracle.forward(inp["qr"], inp["kr"], inp["v"], inp["mu"], inp["var_raw"], inp["prior_logits"],
                         w.causal, w.eps, w.var_floor)
    d = {k: v.to(DEV) for k, v in inp.items()}
    for algo in ("auto", "simt"):
        print("[gpu-case] hypothesis", algo, p, file=sys.stderr, flush=True)
        out = gma.forward(d["qr"], d["kr"], d["v"], d["mu"], d["var_raw"], d["prior_logits"], causal=w.causal,
                          eps=w.eps, var_floor=w.var_floor, algo=algo)
        torch.cuda.synchronize()
        out = out.cpu()
        assert np.all(np.isfinite(out.float().numpy()))
        err = metrics.rowrel(out, ref)
        assert err <= metrics.tol_for(w.dtype), (algo, p, err)
