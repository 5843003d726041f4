"""CPU-only checks of the C ABI (include/gma.h): the library loads, exports every
declared entry point, and rejects invalid calls with the documented status codes
before any HIP call (so these run on a machine without a GPU).  Pointers below are
fake, aligned, non-overlapping addresses: every case fails validation, so none is
ever dereferenced and no kernel is launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gma.h")

binding = pytest.importorskip("gaussian_mixture_sequence_resp_amd.binding")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libgma.so is not built; run __graft_entry__.build()")
    return binding.load_library()


def _header_text():
    return open(HEADER).read()


def _codes():
    txt = _header_text()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"(GMA_OK|GMA_ERR_[A-Z_]+)\s*=\s*(-?\d+)", txt)}


def test_exports_every_declared_symbol(lib):
    txt = re.sub(r"/\*.*?\*/", "", _header_text(), flags=re.S)
    names = set(re.findall(r"\b(gma_[a-z_]+)\s*\(", txt))
    assert names == {"gma_workspace_size", "gma_forward", "gma_forward_timed", "gma_strerror",
                     "gma_version", "gma_workspace_size_cross", "gma_forward_cross",
                     "gma_forward_cross_timed", "gma_memory_workspace_size", "gma_memory",
                     "gma_decode_workspace_size", "gma_decode_step", "gma_stats_workspace_size",
                     "gma_resp_stats", "gma_backward_workspace_size", "gma_backward",
                     "gma_forward_noalloc", "gma_decode_prepared_size", "gma_decode_prepare",
                     "gma_decode_step_prepared"}
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strerror(lib):
    m = re.search(r"#define GMA_VERSION (\d+)", _header_text())
    assert lib.gma_version() == int(m.group(1))
    for code in _codes().values():
        s = binding.strerror(code)
        assert s and s != "unknown status"
    assert binding.strerror(-999) == "unknown status"


class Call:
    """A valid-looking call with fake device addresses; tests perturb one field."""
    BASE = 1 << 32

    def __init__(self, **kw):
        self.desc = binding.make_desc(2, 3, 64, 16, 8, 12, "bf16", 1e-3, "simt")
        for k in ("B", "H", "N", "d_r", "d_v", "K", "dtype", "algo", "var_floor"):
            if k in kw:
                setattr(self.desc, k, kw.pop(k))
        step = 1 << 24
        self.ptr = {n: self.BASE + i * step for i, n in enumerate(
            ["qr", "kr", "v", "mu", "var_raw", "prior", "out", "gamma", "ws"])}
        self.ptr["gamma"] = None
        self.causal, self.eps = 0, 1e-6
        self.ws_bytes = 1 << 40
        for k, val in kw.items():
            if k in self.ptr:
                self.ptr[k] = val
            else:
                setattr(self, k, val)

    def run(self, lib, desc_null=False):
        p = self.ptr
        d = None if desc_null else ctypes.byref(self.desc)
        return lib.gma_forward(p["qr"], p["kr"], p["v"], p["mu"], p["var_raw"], p["prior"],
                               self.causal, self.eps, p["out"], p["gamma"], d, p["ws"],
                               self.ws_bytes, None)

    def run_cross(self, lib, n_k):
        p = self.ptr
        return lib.gma_forward_cross(p["qr"], p["kr"], p["v"], p["mu"], p["var_raw"], p["prior"],
                                     n_k, self.eps, p["out"], p["gamma"], ctypes.byref(self.desc),
                                     p["ws"], self.ws_bytes, None)


C = _codes()


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), "GMA_ERR_BAD_SHAPE"), (dict(K=0), "GMA_ERR_BAD_SHAPE"),
    (dict(d_r=0), "GMA_ERR_BAD_SHAPE"), (dict(d_v=0), "GMA_ERR_BAD_SHAPE"),
    (dict(B=1 << 16, H=1 << 16), "GMA_ERR_BAD_SHAPE"),
    (dict(K=257), "GMA_ERR_UNSUPPORTED"), (dict(d_r=129), "GMA_ERR_UNSUPPORTED"),
    (dict(d_v=129), "GMA_ERR_UNSUPPORTED"), (dict(dtype=7), "GMA_ERR_UNSUPPORTED"),
    (dict(algo=9), "GMA_ERR_UNSUPPORTED"), (dict(algo=2, dtype=0), "GMA_ERR_UNSUPPORTED"),
    (dict(var_floor=float("nan")), "GMA_ERR_BAD_SCALAR"), (dict(var_floor=-1.0), "GMA_ERR_BAD_SCALAR"),
    (dict(eps=-1.0), "GMA_ERR_BAD_SCALAR"), (dict(eps=float("inf")), "GMA_ERR_BAD_SCALAR"),
    (dict(eps=float("nan")), "GMA_ERR_BAD_SCALAR"), (dict(causal=2), "GMA_ERR_BAD_SCALAR"),
    (dict(qr=None), "GMA_ERR_NULL_ARG"), (dict(out=None), "GMA_ERR_NULL_ARG"),
    (dict(prior=None), "GMA_ERR_NULL_ARG"),
    (dict(qr=Call.BASE + 8), "GMA_ERR_ALIGN"), (dict(out=Call.BASE + 6 * (1 << 24) + 4), "GMA_ERR_ALIGN"),
    (dict(mu=Call.BASE + 3 * (1 << 24) + 2), "GMA_ERR_ALIGN"),
    (dict(ws=Call.BASE + 8 * (1 << 24) + 128), "GMA_ERR_ALIGN"),
    (dict(out=Call.BASE), "GMA_ERR_ALIAS"), (dict(gamma=Call.BASE + (1 << 24)), "GMA_ERR_ALIAS"),
    (dict(ws=Call.BASE + 2 * (1 << 24)), "GMA_ERR_ALIAS"),
    (dict(ws_bytes=16), "GMA_ERR_WORKSPACE"), (dict(ws=None), "GMA_ERR_WORKSPACE"),
])
def test_invalid_calls_return_documented_codes(lib, kw, code):
    assert Call(**kw).run(lib) == C[code]


def test_null_descriptor(lib):
    assert Call().run(lib, desc_null=True) == C["GMA_ERR_NULL_ARG"]


def test_empty_problem_is_ok_without_launch(lib):
    # N = 0 (or B = 0): a valid no-op, returns before touching any pointer or the GPU
    assert Call(N=0, qr=None, ws=None).run(lib) == C["GMA_OK"]
    assert Call(B=0).run(lib) == C["GMA_OK"]


def test_workspace_size(lib):
    d = binding.make_desc(2, 3, 64, 16, 8, 12, "bf16", 1e-3, "simt")
    n = binding.workspace_size(d, False)
    assert n > 0 and n % 256 == 0
    # SIMT materialises both responsibility maps: at least 2*B*H*N*K floats
    assert n >= 2 * 2 * 3 * 64 * 12 * 4
    bad = binding.make_desc(2, 3, 64, 16, 8, 999, "bf16", 1e-3, "simt")
    assert binding.workspace_size(bad, False) == 0
    assert lib.gma_workspace_size(None, 0) == 0
    assert binding.workspace_size(binding.make_desc(2, 3, 0, 16, 8, 12, "f32", 1e-3), True) == 0


def test_matrix_core_path_coverage(lib):
    # the matrix-core path takes bf16 with d_r, d_v multiples of 8; an explicit request
    # outside that range is unsupported (workspace 0), AUTO falls back to the SIMT path
    ok = binding.make_desc(2, 3, 64, 64, 64, 128, "bf16", 1e-3, "mfma")
    assert binding.workspace_size(ok, False) > 0 and binding.workspace_size(ok, True) > 0
    for dr, dv in ((100, 64), (64, 100), (5, 7)):
        bad = binding.make_desc(2, 3, 64, dr, dv, 128, "bf16", 1e-3, "mfma")
        assert binding.workspace_size(bad, False) == 0 and binding.workspace_size(bad, True) == 0
        auto = binding.make_desc(2, 3, 64, dr, dv, 128, "bf16", 1e-3, "auto")
        simt = binding.make_desc(2, 3, 64, dr, dv, 128, "bf16", 1e-3, "simt")
        assert binding.workspace_size(auto, False) == binding.workspace_size(simt, False) > 0
    assert binding.workspace_size(binding.make_desc(2, 3, 64, 64, 64, 128, "f32", 1e-3, "mfma"), False) == 0


def test_cross_validation_codes(lib):
    # same checks as gma_forward, sized by N_q for qr/out and n_k for kr/v; no HIP call
    step = 1 << 24
    assert Call().run_cross(lib, -1) == C["GMA_ERR_BAD_SHAPE"]
    assert Call(kr=None).run_cross(lib, 64) == C["GMA_ERR_NULL_ARG"]
    assert Call(eps=-1.0).run_cross(lib, 64) == C["GMA_ERR_BAD_SCALAR"]
    assert Call(v=Call.BASE + 2 * step + 8).run_cross(lib, 64) == C["GMA_ERR_ALIGN"]
    assert Call(ws_bytes=16).run_cross(lib, 64) == C["GMA_ERR_WORKSPACE"]
    # a long key sequence: kr (2*3*n_k*16 bf16 = 192 n_k bytes) and v (96 n_k bytes) grow
    # into `out`, 5 and 4 slots later
    assert Call().run_cross(lib, (4 * step) // 96 + 1) == C["GMA_ERR_ALIAS"]
    # empty query side: a no-op that touches nothing
    assert Call(N=0, qr=None, ws=None).run_cross(lib, 99) == C["GMA_OK"]
    # empty key side: kr and v may be NULL (validation then fails later, on the workspace)
    assert Call(kr=None, v=None, ws_bytes=16).run_cross(lib, 0) == C["GMA_ERR_WORKSPACE"]
    assert Call(kr=None, v=None, ws_bytes=16).run_cross(lib, 1) == C["GMA_ERR_NULL_ARG"]


def test_cross_workspace_size(lib):
    d = binding.make_desc(2, 3, 64, 16, 8, 12, "bf16", 1e-3, "simt")
    # SIMT materialises Gamma_Q (B*H*Nq*K) and Gamma_K (B*H*Nk*K) as float32
    small, big = binding.workspace_size_cross(d, 10), binding.workspace_size_cross(d, 1000)
    assert 0 < small < big and big >= 2 * 3 * (64 + 1000) * 12 * 4
    assert binding.workspace_size_cross(d, 64) == binding.workspace_size(d, False)
    assert binding.workspace_size_cross(d, -1) == 0
    assert binding.workspace_size_cross(d, 0) > 0
    dm = binding.make_desc(2, 3, 64, 64, 64, 128, "bf16", 1e-3, "mfma")
    assert binding.workspace_size_cross(dm, 5000) > 0
    assert binding.workspace_size_cross(dm, 64) == binding.workspace_size(dm, False)


def test_memory_and_decode_validation(lib):
    vp = ctypes.c_void_p
    lib.gma_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp,
                                    ctypes.POINTER(binding.GmaDesc), vp, ctypes.c_size_t, vp]
    lib.gma_memory.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(binding.GmaDesc), vp, ctypes.c_size_t, vp]
    step = 1 << 24
    P = [Call.BASE + i * step for i in range(10)]  # qr kr v mu var_raw prior state out ws, spare

    def dec(desc, eps=1e-6, **kw):
        p = dict(qr=P[0], kr=P[1], v=P[2], mu=P[3], vr=P[4], pr=P[5], st=P[6], out=P[7], ws=P[8], nb=1 << 40)
        p.update(kw)
        return lib.gma_decode_step(p["qr"], p["kr"], p["v"], p["mu"], p["vr"], p["pr"], p["st"], eps, p["out"],
                                   ctypes.byref(desc), p["ws"], p["nb"], None)

    def mem(desc, **kw):
        p = dict(kr=P[1], v=P[2], mu=P[3], vr=P[4], pr=P[5], st=P[6], ws=P[8], nb=1 << 40)
        p.update(kw)
        return lib.gma_memory(p["kr"], p["v"], p["mu"], p["vr"], p["pr"], p["st"], ctypes.byref(desc), p["ws"],
                              p["nb"], None)

    d1 = binding.make_desc(2, 3, 1, 16, 8, 12, "bf16", 1e-3, "auto")
    assert dec(binding.make_desc(2, 3, 2, 16, 8, 12, "bf16", 1e-3)) == C["GMA_ERR_BAD_SHAPE"]
    assert dec(binding.make_desc(2, 3, 1, 16, 8, 12, "bf16", 1e-3, "mfma")) == C["GMA_ERR_UNSUPPORTED"]
    assert dec(d1, eps=-1.0) == C["GMA_ERR_BAD_SCALAR"]
    assert dec(d1, st=None) == C["GMA_ERR_NULL_ARG"]
    assert dec(d1, st=P[6] + 2) == C["GMA_ERR_ALIGN"]
    assert dec(d1, out=P[6]) == C["GMA_ERR_ALIAS"]
    assert dec(d1, st=P[0]) == C["GMA_ERR_ALIAS"]
    assert dec(binding.make_desc(0, 3, 1, 16, 8, 12, "bf16", 1e-3), qr=None) == C["GMA_OK"]
    # the decode step needs no workspace: one kernel, its reductions in LDS
    assert binding.load_library().gma_decode_workspace_size(ctypes.byref(d1)) == 0
    dm = binding.make_desc(2, 3, 64, 16, 8, 12, "bf16", 1e-3, "auto")
    assert mem(dm, st=None) == C["GMA_ERR_NULL_ARG"]
    assert mem(dm, kr=None) == C["GMA_ERR_NULL_ARG"]
    assert mem(dm, st=P[1]) == C["GMA_ERR_ALIAS"]
    assert mem(dm, nb=8) == C["GMA_ERR_WORKSPACE"]
    assert mem(binding.make_desc(2, 3, 64, 100, 8, 12, "bf16", 1e-3, "mfma")) == C["GMA_ERR_UNSUPPORTED"]
    # an empty prefix needs no kr / v (the state is still written: fails here on the workspace)
    assert mem(binding.make_desc(2, 3, 0, 16, 8, 12, "bf16", 1e-3), kr=None, v=None, nb=8) == C["GMA_ERR_WORKSPACE"]
    assert binding.load_library().gma_memory_workspace_size(ctypes.byref(dm)) > 0


def test_prepared_decode_validation(lib):
    # every call below fails validation (or is an empty no-op) before any HIP call
    vp = ctypes.c_void_p
    lib.gma_decode_prepare.argtypes = [vp, vp, vp, vp, ctypes.c_size_t, ctypes.POINTER(binding.GmaDesc), vp]
    lib.gma_decode_step_prepared.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp,
                                             ctypes.POINTER(binding.GmaDesc), vp]
    step = 1 << 24
    P = [Call.BASE + i * step for i in range(8)]  # mu var_raw prior prepared qr kr v state; out spare

    def prep(desc, **kw):
        p = dict(mu=P[0], vr=P[1], pr=P[2], pp=P[3], nb=1 << 30)
        p.update(kw)
        return lib.gma_decode_prepare(p["mu"], p["vr"], p["pr"], p["pp"], p["nb"], ctypes.byref(desc), None)

    def step_(desc, eps=1e-6, **kw):
        p = dict(qr=P[4], kr=P[5], v=P[6], pp=P[3], st=P[7], out=P[7] + step // 2)
        p.update(kw)
        return lib.gma_decode_step_prepared(p["qr"], p["kr"], p["v"], p["pp"], p["st"], eps, p["out"],
                                            ctypes.byref(desc), None)

    d1 = binding.make_desc(2, 3, 1, 16, 8, 12, "bf16", 1e-3)
    need = int(lib.gma_decode_prepared_size(ctypes.byref(d1)))
    # float32 (mu, lambda) pairs for bf16 inputs, float64 for float32, and one float64 constant per component
    assert need == 3 * 12 * 16 * 8 + 3 * 12 * 8
    assert int(lib.gma_decode_prepared_size(ctypes.byref(binding.make_desc(2, 3, 1, 16, 8, 12, "f32", 1e-3)))) \
        == 3 * 12 * 16 * 16 + 3 * 12 * 8
    assert lib.gma_decode_prepared_size(ctypes.byref(binding.make_desc(2, 3, 1, 16, 8, 300, "bf16", 1e-3))) == 0
    assert prep(d1, nb=need - 1) == C["GMA_ERR_WORKSPACE"]
    assert prep(d1, pp=None) == C["GMA_ERR_NULL_ARG"]
    assert prep(d1, pp=P[3] + 64) == C["GMA_ERR_ALIGN"]
    assert prep(d1, pp=P[0]) == C["GMA_ERR_ALIAS"]
    assert prep(binding.make_desc(2, 3, 1, 16, 8, 12, "bf16", -1.0)) == C["GMA_ERR_BAD_SCALAR"]
    assert prep(binding.make_desc(2, 0, 1, 16, 8, 12, "bf16", 1e-3), mu=None) == C["GMA_OK"]
    assert step_(binding.make_desc(2, 3, 2, 16, 8, 12, "bf16", 1e-3)) == C["GMA_ERR_BAD_SHAPE"]
    assert step_(binding.make_desc(2, 3, 1, 16, 8, 12, "bf16", 1e-3, "mfma")) == C["GMA_ERR_UNSUPPORTED"]
    assert step_(d1, eps=float("nan")) == C["GMA_ERR_BAD_SCALAR"]
    assert step_(d1, pp=None) == C["GMA_ERR_NULL_ARG"]
    assert step_(d1, pp=P[3] + 16) == C["GMA_ERR_ALIGN"]
    assert step_(d1, st=P[3]) == C["GMA_ERR_ALIAS"]
    assert step_(d1, out=P[4]) == C["GMA_ERR_ALIAS"]
    assert step_(binding.make_desc(0, 3, 1, 16, 8, 12, "bf16", 1e-3), qr=None) == C["GMA_OK"]


def test_stats_validation(lib):
    # every call below fails validation (or is an empty no-op) before any HIP call
    vp = ctypes.c_void_p
    lib.gma_resp_stats.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(binding.GmaDesc), vp,
                                   ctypes.c_size_t, vp]
    step = 1 << 24
    P = [Call.BASE + i * step for i in range(12)]  # x mu var_raw prior hard counts usage used entropy ws

    def call(desc, **kw):
        p = dict(x=P[0], mu=P[1], vr=P[2], pr=P[3], hard=P[4], counts=P[5], usage=P[6], used=P[7], ent=P[8],
                 ws=P[9], nb=1 << 40)
        p.update(kw)
        return lib.gma_resp_stats(p["x"], p["mu"], p["vr"], p["pr"], p["hard"], p["counts"], p["usage"],
                                  p["used"], p["ent"], ctypes.byref(desc), p["ws"], p["nb"], None)

    d = binding.make_desc(2, 3, 64, 16, 1, 12, "bf16", 1e-3, "auto")
    assert call(binding.make_desc(0, 3, 64, 16, 1, 12, "bf16", 1e-3), x=None, counts=None) == C["GMA_OK"]
    assert call(d, counts=None) == C["GMA_ERR_NULL_ARG"]
    assert call(d, ent=None) == C["GMA_ERR_NULL_ARG"]
    assert call(d, x=None) == C["GMA_ERR_NULL_ARG"]
    assert call(d, x=P[0] + 2) == C["GMA_ERR_ALIGN"]
    assert call(d, counts=P[5] + 2) == C["GMA_ERR_ALIGN"]
    assert call(d, ws=P[9] + 16) == C["GMA_ERR_ALIGN"]
    assert call(binding.make_desc(2, 3, 64, 16, 1, 12, "f32", 1e-3, "mfma")) == C["GMA_ERR_UNSUPPORTED"]
    assert call(binding.make_desc(2, 3, 64, 12, 1, 12, "bf16", 1e-3, "mfma")) == C["GMA_ERR_UNSUPPORTED"]
    assert call(binding.make_desc(2, 3, 64, 16, 1, 300, "bf16", 1e-3)) == C["GMA_ERR_UNSUPPORTED"]
    assert call(d, nb=8) == C["GMA_ERR_WORKSPACE"]
    assert call(d, ws=None) == C["GMA_ERR_WORKSPACE"]
    assert call(d, usage=P[5]) == C["GMA_ERR_ALIAS"]
    assert call(d, hard=P[0]) == C["GMA_ERR_ALIAS"]
    assert call(d, ws=P[1]) == C["GMA_ERR_ALIAS"]
    sz = binding.load_library().gma_stats_workspace_size
    sz.argtypes = [ctypes.POINTER(binding.GmaDesc)]
    sz.restype = ctypes.c_size_t
    assert sz(ctypes.byref(d)) > 0
    assert sz(ctypes.byref(binding.make_desc(2, 3, 64, 16, 1, 12, "f32", 1e-3))) > 0
    assert sz(ctypes.byref(binding.make_desc(0, 3, 64, 16, 1, 12, "bf16", 1e-3))) == 0
    assert sz(ctypes.byref(binding.make_desc(2, 3, 64, 12, 1, 12, "bf16", 1e-3, "mfma"))) == 0


def test_backward_validation(lib):
    # every call below fails validation (or is an empty no-op) before any HIP call
    vp = ctypes.c_void_p
    lib.gma_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_float, vp, vp, vp, vp, vp, vp,
                                 ctypes.POINTER(binding.GmaDesc), vp, ctypes.c_size_t, vp]
    step = 1 << 24
    P = [Call.BASE + i * step for i in range(16)]
    names = ("qr", "kr", "v", "mu", "vr", "pr", "do", "dq", "dk", "dv", "dmu", "dvr", "dpr", "ws")

    def call(desc, causal=0, eps=1e-6, **kw):
        p = dict(zip(names, P))
        p["nb"] = 1 << 40
        p.update(kw)
        return lib.gma_backward(p["qr"], p["kr"], p["v"], p["mu"], p["vr"], p["pr"], p["do"], causal, eps, p["dq"],
                                p["dk"], p["dv"], p["dmu"], p["dvr"], p["dpr"], ctypes.byref(desc), p["ws"], p["nb"],
                                None)

    d = binding.make_desc(2, 3, 64, 16, 8, 12, "bf16", 1e-3, "auto")
    assert call(binding.make_desc(0, 3, 64, 16, 8, 12, "bf16", 1e-3), qr=None, dmu=None) == C["GMA_OK"]
    assert call(d, causal=2) == C["GMA_ERR_BAD_SCALAR"]
    assert call(d, eps=-1.0) == C["GMA_ERR_BAD_SCALAR"]
    assert call(d, dmu=None) == C["GMA_ERR_NULL_ARG"]
    assert call(d, do=None) == C["GMA_ERR_NULL_ARG"]
    assert call(d, dq=P[7] + 8) == C["GMA_ERR_ALIGN"]
    assert call(d, dpr=P[12] + 2) == C["GMA_ERR_ALIGN"]
    assert call(binding.make_desc(2, 3, 64, 16, 8, 12, "bf16", 1e-3, "mfma")) == C["GMA_ERR_UNSUPPORTED"]
    assert call(d, nb=8) == C["GMA_ERR_WORKSPACE"]
    assert call(d, dq=P[0]) == C["GMA_ERR_ALIAS"]
    assert call(d, dk=P[7]) == C["GMA_ERR_ALIAS"]
    assert call(d, dv=P[6]) == C["GMA_ERR_ALIAS"]
    assert call(d, ws=P[3]) == C["GMA_ERR_ALIAS"]
    sz = binding.load_library().gma_backward_workspace_size
    assert sz(ctypes.byref(d), 0) > 0 and sz(ctypes.byref(d), 1) > 0
    assert sz(ctypes.byref(d), 2) == 0
    assert sz(ctypes.byref(binding.make_desc(2, 3, 64, 16, 8, 12, "bf16", 1e-3, "mfma")), 0) == 0
    # 2 B N above INT32_MAX (B H N itself within it): the row passes would overflow their
    # 32-bit row index, so the shape is refused with a workspace size of 0
    big = binding.make_desc(1 << 15, 1, (1 << 15) + 1, 16, 8, 12, "bf16", 1e-3, "auto")
    assert sz(ctypes.byref(big), 0) == 0 and sz(ctypes.byref(big), 1) == 0
    assert call(big) == C["GMA_ERR_UNSUPPORTED"]
    ok = binding.make_desc(1 << 14, 1, (1 << 16) - 1, 16, 8, 12, "bf16", 1e-3, "auto")  # 2 B N < 2^31
    assert sz(ctypes.byref(ok), 0) > 0


# ---- Python binding: every tensor argument is validated before any library call, so a
# mismatched shape, dtype or device raises GMAError instead of letting a kernel read or write
# out of bounds (or dereference a host pointer).  All tensors here are CPU tensors: the shape
# and dtype checks fire first, and a call that passes them fails on the device check.

torch = pytest.importorskip("torch")


def _fwd_inputs(B=2, H=3, N=16, dr=8, dv=8, K=4, dt=None):
    dt = dt or torch.bfloat16
    return dict(qr=torch.zeros(B, H, N, dr, dtype=dt), kr=torch.zeros(B, H, N, dr, dtype=dt),
                v=torch.zeros(B, H, N, dv, dtype=dt), mu=torch.zeros(H, K, dr),
                var_raw=torch.zeros(H, K, dr), prior_logits=torch.zeros(H, K))


def _code(fn, *a, **kw):
    with pytest.raises(binding.GMAError) as ei:
        fn(*a, **kw)
    return ei.value.code


@pytest.mark.parametrize("field,bad", [
    ("kr", lambda t: t[:, :, :-1].contiguous()),          # shorter key sequence
    ("kr", lambda t: t[..., :-1].contiguous()),           # other routing dim
    ("v", lambda t: t[:, :, :-2].contiguous()),           # fewer value rows
    ("mu", lambda t: t[:, :-1].contiguous()),             # other K than var_raw
    ("var_raw", lambda t: t[:, :, :-1].contiguous()),     # other d_r
    ("prior_logits", lambda t: t[:, :-1].contiguous()),   # other K
    ("mu", lambda t: t[:-1].contiguous()),                # fewer heads
])
def test_binding_rejects_shape_mismatch(field, bad):
    inp = _fwd_inputs()
    inp[field] = bad(inp[field])
    assert _code(binding.forward, **inp) == -2
    if field not in ("kr",):
        assert _code(binding.backward, **inp, dout=torch.zeros(2, 3, 16, 8, dtype=torch.bfloat16),
                     causal=False) == -2


@pytest.mark.parametrize("field,dt", [("v", torch.float32), ("kr", torch.float32), ("mu", torch.bfloat16),
                                      ("var_raw", torch.float64), ("prior_logits", torch.bfloat16)])
def test_binding_rejects_dtype_mismatch(field, dt):
    inp = _fwd_inputs()
    inp[field] = inp[field].to(dt)
    assert _code(binding.forward, **inp) == -3
    assert _code(binding.backward, **inp, dout=torch.zeros(2, 3, 16, 8, dtype=torch.bfloat16), causal=True) == -3


def test_binding_rejects_bad_outputs_and_buffers():
    inp = _fwd_inputs()
    assert _code(binding.forward, **inp, out=torch.zeros(2, 3, 16, 7, dtype=torch.bfloat16)) == -2
    assert _code(binding.forward, **inp, out=torch.zeros(2, 3, 16, 8)) == -3
    assert _code(binding.forward, **inp, gamma_out=torch.zeros(2, 2, 3, 16, 5)) == -2
    assert _code(binding.forward, **inp, gamma_out=torch.zeros(2, 2, 3, 16, 4, dtype=torch.float64)) == -3
    assert _code(binding.forward, **inp, workspace=torch.zeros(16, dtype=torch.float32)) == -3
    assert _code(binding.backward, **inp, dout=torch.zeros(2, 3, 15, 8, dtype=torch.bfloat16), causal=False) == -2
    # cross: keys of another length are fine, value rows must match the keys
    x = _fwd_inputs()
    x["kr"] = torch.zeros(2, 3, 40, 8, dtype=torch.bfloat16)
    x["v"] = torch.zeros(2, 3, 39, 8, dtype=torch.bfloat16)
    assert _code(binding.forward_cross, **x) == -2
    x["v"] = torch.zeros(2, 3, 40, 8, dtype=torch.bfloat16)
    assert _code(binding.forward_cross, **x, gamma_out=torch.zeros(2 * 3 * 16 * 4)) == -2
    # memory, decode and statistics
    m = _fwd_inputs()
    assert _code(binding.memory, m["kr"], m["v"], m["mu"], m["var_raw"], m["prior_logits"],
                 state=torch.zeros(2, 3, 4, 8)) == -2
    assert _code(binding.decode_step, m["qr"][:, :, :1], m["kr"][:, :, :1], m["v"][:, :, :1], m["mu"],
                 m["var_raw"], m["prior_logits"], torch.zeros(2, 3, 4, 8)) == -2
    assert _code(binding.decode_step, m["qr"][:, :, :2], m["kr"][:, :, :1], m["v"][:, :, :1], m["mu"],
                 m["var_raw"], m["prior_logits"], torch.zeros(2, 3, 4, 9)) == -2
    assert _code(binding.resp_stats, m["kr"], m["mu"][:, :, :4].contiguous(), m["var_raw"],
                 m["prior_logits"]) == -2


def test_binding_rejects_host_tensors():
    """Well-formed arguments that live in host memory: refused before the library sees a
    host pointer (which a kernel would fault on)."""
    inp = _fwd_inputs()
    assert _code(binding.forward, **inp) == binding.GMA_ERR_DEVICE
    assert _code(binding.forward_cross, **inp) == binding.GMA_ERR_DEVICE
    assert _code(binding.backward, **inp, dout=torch.zeros(2, 3, 16, 8, dtype=torch.bfloat16),
                 causal=False) == binding.GMA_ERR_DEVICE
    assert _code(binding.memory, inp["kr"], inp["v"], inp["mu"], inp["var_raw"],
                 inp["prior_logits"]) == binding.GMA_ERR_DEVICE
    assert _code(binding.resp_stats, inp["kr"], inp["mu"], inp["var_raw"],
                 inp["prior_logits"]) == binding.GMA_ERR_DEVICE
    assert _code(binding.decode_step, inp["qr"][:, :, :1], inp["kr"][:, :, :1], inp["v"][:, :, :1], inp["mu"],
                 inp["var_raw"], inp["prior_logits"], torch.zeros(2, 3, 4, 9)) == binding.GMA_ERR_DEVICE


def test_noalloc_validation(lib):
    """gma_forward_noalloc: same checks as gma_forward, then GMA_ERR_TOO_LARGE for a call whose
    workspace exceeds the static scratch -- all before any HIP call (fake pointers here)."""
    cap = int(re.search(r"#define GMA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", _header_text()).group(1)) << 20
    vp = ctypes.c_void_p
    step = 1 << 28
    P = [Call.BASE + i * step for i in range(8)]

    def call(desc, causal=0, eps=1e-6, **kw):
        p = dict(zip(("qr", "kr", "v", "mu", "vr", "pr", "out"), P))
        p.update(kw)
        return lib.gma_forward_noalloc(p["qr"], p["kr"], p["v"], p["mu"], p["vr"], p["pr"], causal, eps, p["out"],
                                       None, ctypes.byref(desc), None)

    d = binding.make_desc(2, 3, 64, 16, 8, 12, "bf16", 1e-3, "auto")
    assert call(d, causal=2) == C["GMA_ERR_BAD_SCALAR"]
    assert call(d, out=None) == C["GMA_ERR_NULL_ARG"]
    assert call(d, out=P[0]) == C["GMA_ERR_ALIAS"]
    assert call(d, qr=P[0] + 8) == C["GMA_ERR_ALIGN"]
    assert call(binding.make_desc(0, 3, 64, 16, 8, 12, "bf16", 1e-3)) == C["GMA_OK"]  # empty: no launch
    # a shape whose workspace is beyond the static scratch
    big = binding.make_desc(64, 8, 8192, 64, 64, 128, "bf16", 1e-3, "simt")
    need = binding.workspace_size(big, False)
    assert need > cap
    big_ptrs = {n: Call.BASE + i * (1 << 34) for i, n in enumerate(("qr", "kr", "v", "mu", "vr", "pr", "out"))}
    assert call(big, **big_ptrs) == C["GMA_ERR_TOO_LARGE"]
    assert "GMA_NOALLOC_SCRATCH_BYTES" in binding.strerror(C["GMA_ERR_TOO_LARGE"])
