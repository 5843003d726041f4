"""GPU parity of the causal memory (prefill) and the single-token decode step against the
fp64 oracle, through the C ABI (gma_memory, gma_decode_step, and gma_decode_prepare +
gma_decode_step_prepared).

Core mechanism item 3 read as a recurrence: decoding positions t = s..N-1 one at a time
from the memory of positions 0..s-1 reproduces rows s..N-1 of the causal forward.  Gate:
row-normwise relative error <= 1e-5 (float32 inputs), <= 2e-2 (bf16 inputs); the memory
itself is compared row by row the same way.
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


def _say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def _run(inp, w, split, algo="auto", prepared=False):
    """Memory of positions [0, split), then decode steps for the rest (on the raw parameters,
    or on parameters prepared once); returns (outs, state)."""
    d = {k: x.to(DEV) for k, x in inp.items()}
    state = gma.memory(d["kr"][:, :, :split].contiguous(), d["v"][:, :, :split].contiguous(), d["mu"],
                       d["var_raw"], d["prior_logits"], var_floor=w.var_floor, algo=algo)
    params = gma.decode_prepare(d["mu"], d["var_raw"], d["prior_logits"], dtype=w.dtype,
                                var_floor=w.var_floor) if prepared else None
    outs = []
    for t in range(split, w.N):
        sl = slice(t, t + 1)
        if prepared:
            outs.append(gma.decode_step_prepared(d["qr"][:, :, sl], d["kr"][:, :, sl], d["v"][:, :, sl], params,
                                                 state, eps=w.eps))
        else:
            outs.append(gma.decode_step(d["qr"][:, :, sl], d["kr"][:, :, sl], d["v"][:, :, sl], d["mu"],
                                        d["var_raw"], d["prior_logits"], state, eps=w.eps, var_floor=w.var_floor))
    torch.cuda.synchronize()
    out = torch.cat(outs, dim=2).cpu() if outs else None
    return out, state.cpu()


DECODE = [
    # (N, K, d_r, d_v, split)
    (40, 256, 64, 64, 0), (17, 5, 3, 7, 9), (33, 128, 128, 128, 20), (64, 33, 24, 40, 63), (1, 1, 8, 8, 0),
    # bf16 prefills of these run on the causal responsibilities + totals kernels (coefficient
    # blocks too large for the fused write kernel), ragged in positions and components
    (300, 256, 64, 64, 250), (200, 200, 40, 24, 130),
]


@pytest.mark.parametrize("prepared", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,K,dr,dv,split", DECODE)
def test_memory_then_decode_matches_causal_forward(N, K, dr, dv, split, dtype, prepared):
    w = WORKLOADS[3].with_(B=2, H=3, N=N, K=K, d_r=dr, d_v=dv, dtype=dtype, seed=51 + N + K)
    inp = make_inputs(w)
    _say("decode", dtype, dict(N=N, K=K, dr=dr, dv=dv, split=split, seed=w.seed, prepared=prepared))
    out, state = _run(inp, w, split, prepared=prepared)
    ref = oracle.forward(inp["qr"], inp["kr"], inp["v"], inp["mu"], inp["var_raw"], inp["prior_logits"], True,
                         w.eps, w.var_floor)
    tol = metrics.tol_for(dtype)
    if split < N:
        assert np.all(np.isfinite(out.float().numpy()))
        err = metrics.rowrel(out, ref[:, :, split:])
        assert err <= tol, (err, metrics.globalrel(out, ref[:, :, split:]))
    ref_state = oracle.memory(inp["kr"], inp["v"], inp["mu"], inp["var_raw"], inp["prior_logits"], w.var_floor)
    assert metrics.rowrel(state, ref_state) <= tol


@pytest.mark.parametrize("K", [256, 128])
@pytest.mark.parametrize("algo", ["simt", "auto", "mfma"])
def test_memory_long_prefix(algo, K):
    # the prefill on the matrix cores (bf16; K = 128 the fused write kernel, K = 256 the
    # causal responsibilities + totals kernels) and on the SIMT path
    w = WORKLOADS[3].with_(B=2, H=2, N=2048 + 77, K=K, seed=61)
    inp = make_inputs(w)
    _say("memory long prefix", algo, w)
    d = {k: x.to(DEV) for k, x in inp.items()}
    state = gma.memory(d["kr"], d["v"], d["mu"], d["var_raw"], d["prior_logits"], var_floor=w.var_floor,
                       algo=algo)
    torch.cuda.synchronize()
    ref = oracle.memory(inp["kr"], inp["v"], inp["mu"], inp["var_raw"], inp["prior_logits"], w.var_floor)
    err = metrics.rowrel(state.cpu(), ref)
    _say("memory long prefix rowrel", err)
    assert err <= metrics.tol_for(w.dtype)
    # the normaliser column: z_k sums to the number of positions
    np.testing.assert_allclose(state.cpu()[..., -1].sum(-1).numpy(), w.N, rtol=1e-4)


@pytest.mark.parametrize("algo", ["auto", "mfma"])
def test_memory_wide_routing(algo):
    # 256 components of 128 routing dims: the prefill runs the component-parallel
    # responsibilities on the key side only (one side per launch), then the totals kernels;
    # a ragged prefix over several workgroup parts
    w = WORKLOADS[3].with_(B=2, H=2, N=3000 + 45, K=256, d_r=128, d_v=64, seed=62)
    inp = make_inputs(w)
    _say("memory wide routing", algo, w)
    d = {k: x.to(DEV) for k, x in inp.items()}
    state = gma.memory(d["kr"], d["v"], d["mu"], d["var_raw"], d["prior_logits"], var_floor=w.var_floor,
                       algo=algo)
    torch.cuda.synchronize()
    ref = oracle.memory(inp["kr"], inp["v"], inp["mu"], inp["var_raw"], inp["prior_logits"], w.var_floor)
    err = metrics.rowrel(state.cpu(), ref)
    _say("memory wide routing rowrel", err)
    assert err <= metrics.tol_for(w.dtype)
    np.testing.assert_allclose(state.cpu()[..., -1].sum(-1).numpy(), w.N, rtol=1e-4)


def test_memory_of_empty_prefix_is_zero():
    w = WORKLOADS[3].with_(B=2, H=2, N=0, seed=62)
    inp = make_inputs(w)
    d = {k: x.to(DEV) for k, x in inp.items()}
    for algo in ("simt", "auto", "mfma"):
        state = torch.full((2, 2, w.K, w.d_v + 1), 7.0, device=DEV)
        gma.memory(d["kr"], d["v"], d["mu"], d["var_raw"], d["prior_logits"], var_floor=w.var_floor, state=state,
                   algo=algo)
        torch.cuda.synchronize()
        assert torch.count_nonzero(state) == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_with_parameters_not_16_byte_aligned(dtype):
    # mu and var_raw views starting one float into their buffers (4-byte aligned, as the ABI
    # allows): the decode kernel takes its scalar-load path; same results as aligned copies
    w = WORKLOADS[3].with_(B=2, H=3, N=6, K=40, d_r=32, d_v=16, dtype=dtype, seed=63)
    inp = make_inputs(w)
    d = {k: x.to(DEV) for k, x in inp.items()}
    _say("decode unaligned parameters", dtype)

    def shifted(x):
        buf = torch.zeros(x.numel() + 1, dtype=x.dtype, device=DEV)
        buf[1:] = x.reshape(-1)
        return buf[1:].view(x.shape)

    mu_s, vr_s = shifted(d["mu"]), shifted(d["var_raw"])
    assert mu_s.data_ptr() % 16 != 0 and vr_s.data_ptr() % 16 != 0
    outs = []
    for mu, vr in ((d["mu"], d["var_raw"]), (mu_s, vr_s)):
        state = gma.memory(d["kr"][:, :, :3].contiguous(), d["v"][:, :, :3].contiguous(), mu, vr, d["prior_logits"],
                           var_floor=w.var_floor)
        o = [gma.decode_step(d["qr"][:, :, t:t + 1], d["kr"][:, :, t:t + 1], d["v"][:, :, t:t + 1], mu, vr,
                             d["prior_logits"], state, eps=w.eps, var_floor=w.var_floor) for t in range(3, 6)]
        outs.append(torch.cat(o, dim=2).cpu())
    ref = oracle.forward(inp["qr"], inp["kr"], inp["v"], inp["mu"], inp["var_raw"], inp["prior_logits"], True,
                         w.eps, w.var_floor)
    for o in outs:
        assert metrics.rowrel(o, ref[:, :, 3:]) <= metrics.tol_for(dtype)


@pytest.mark.parametrize("prepared", [False, True])
def test_decode_full_size_sampled_heads(prepared):
    """Prefill and decode at the benchmark's shape (the causal LM workload: B=16, H=8, K=256,
    d=64, a prefix of 2048 positions, then 8 decode steps, all (b, h) in each launch): the
    memory and the step outputs of heads 0 and H-1 (all batch elements) against the oracle
    run on those heads alone."""
    base = WORKLOADS[3]
    steps = 8
    w = base.with_(N=base.N + steps)
    inp = make_inputs(w)
    _say("decode full size", w.name, dict(B=w.B, H=w.H, prefix=base.N, steps=steps, K=w.K, prepared=prepared))
    out, state = _run(inp, w, base.N, prepared=prepared)
    tol = metrics.tol_for(w.dtype)
    for h in (0, w.H - 1):
        sub = {k: (x[:, h:h + 1].contiguous() if k in ("qr", "kr", "v") else x[h:h + 1].contiguous())
               for k, x in inp.items()}
        ref = oracle.forward(sub["qr"], sub["kr"], sub["v"], sub["mu"], sub["var_raw"], sub["prior_logits"], True,
                             w.eps, w.var_floor)
        err = metrics.rowrel(out[:, h:h + 1], ref[:, :, base.N:])
        ref_state = oracle.memory(sub["kr"], sub["v"], sub["mu"], sub["var_raw"], sub["prior_logits"], w.var_floor)
        serr = metrics.rowrel(state[:, h:h + 1], ref_state)
        _say("decode full size head", h, f"out {err:.2e}", f"state after the steps {serr:.2e}")
        assert err <= tol and serr <= tol, (h, err, serr)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prepared_step_matches_raw_step(dtype):
    """The prepared and the raw decode step are two evaluations of the same step: after the
    same prefill, their outputs and states agree to the dtype's gate, for every (b, h) of a
    batch large enough that the prepared step splits each (b, h) over several column groups
    (B*H = 24, d_v = 96)."""
    w = WORKLOADS[3].with_(B=4, H=6, N=70, K=256, d_r=64, d_v=96, dtype=dtype, seed=64)
    inp = make_inputs(w)
    _say("prepared vs raw", dtype)
    raw, sraw = _run(inp, w, 60)
    prep, sprep = _run(inp, w, 60, prepared=True)
    tol = metrics.tol_for(dtype)
    assert metrics.rowrel(prep, raw) <= tol
    assert metrics.rowrel(sprep, sraw) <= tol
    ref = oracle.forward(inp["qr"], inp["kr"], inp["v"], inp["mu"], inp["var_raw"], inp["prior_logits"], True,
                         w.eps, w.var_floor)
    assert metrics.rowrel(prep, ref[:, :, 60:]) <= tol


@pytest.mark.parametrize("prepared", [False, True])
def test_decode_steps_replayed_from_a_graph(prepared):
    """Decode steps captured in a HIP graph (the way a serving loop launches them; neither
    step allocates or clears memory) and replayed three times, each replay from the same
    prefill, eager work and synchronisation in between: every replay's outputs and state
    equal the eager run's bitwise (the same kernels on the same inputs)."""
    w = WORKLOADS[3].with_(B=4, H=4, N=40, seed=65)
    inp = make_inputs(w)
    d = {k: x.to(DEV) for k, x in inp.items()}
    split, steps = 32, 8
    _say("decode graph replay", dict(prepared=prepared, steps=steps))
    state = torch.empty((w.B, w.H, w.K, w.d_v + 1), dtype=torch.float32, device=DEV)
    params = gma.decode_prepare(d["mu"], d["var_raw"], d["prior_logits"], dtype=w.dtype,
                                var_floor=w.var_floor) if prepared else None
    rows = [(d["qr"][:, :, t:t + 1].contiguous(), d["kr"][:, :, t:t + 1].contiguous(),
             d["v"][:, :, t:t + 1].contiguous()) for t in range(split, split + steps)]
    outs = [torch.empty((w.B, w.H, 1, w.d_v), dtype=d["qr"].dtype, device=DEV) for _ in range(steps)]

    def prefill():
        gma.memory(d["kr"][:, :, :split].contiguous(), d["v"][:, :, :split].contiguous(), d["mu"], d["var_raw"],
                   d["prior_logits"], var_floor=w.var_floor, state=state)

    def run_steps():
        for i, (q, k, v) in enumerate(rows):
            if prepared:
                gma.decode_step_prepared(q, k, v, params, state, eps=w.eps, out=outs[i])
            else:
                gma.decode_step(q, k, v, d["mu"], d["var_raw"], d["prior_logits"], state, eps=w.eps,
                                var_floor=w.var_floor, out=outs[i])

    prefill()
    run_steps()
    torch.cuda.synchronize()
    eager_out = torch.cat([o.clone() for o in outs], dim=2).cpu()
    eager_state = state.clone().cpu()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        prefill()
        run_steps()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_steps()
    for rep in range(3):
        prefill()
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = torch.cat([o.clone() for o in outs], dim=2).cpu()
        assert torch.equal(got, eager_out), rep
        assert torch.equal(state.cpu(), eager_state), rep
