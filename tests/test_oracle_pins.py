"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Source: "Gaussian Mixture Attention" (arXiv 2606.18283), gist.science summaries,
section "Core mechanism": responsibilities are standard GMM posteriors with
diagonal covariances (item 1); the write/read equations and the associativity
argument (item 2); softplus variances, softmax priors and the causal prefix-sum
variant (item 3).  Section "Contributions", theoretical analysis: the induced
affinity is non-negative with rank <= K.

Each pin is chosen so that a plausible slip in the oracle (a dropped constant,
a sign, a swapped operand, an off-by-one in the causal boundary, softplus on the
wrong quantity) fails at least one of them:
  * log joint vs scipy's multivariate normal log-pdf  (constants, signs, softplus)
  * posteriors vs scikit-learn's diagonal GaussianMixture.predict_proba
  * 1-D two-component posterior vs the textbook logistic / quadratic discriminant
  * mixing vs an independent N x N brute force (associativity, causal mask)
  * closed forms: K = 1 mean / prefix mean, identical components
  * invariants: rows on the simplex, rank(A) <= K, semiseparable causal rank,
    bound by max|v|, linearity in V, prior shift invariance, permutation
    equivariance, exact causality.
"""
import numpy as np
import pytest
import scipy.special
import scipy.stats
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle
from tests import metrics


def _params(rng, K, d, mu_std=1.0, vr_std=0.5, p_std=1.0):
    mu = rng.normal(0.0, mu_std, size=(K, d))
    vr = rng.normal(0.0, vr_std, size=(K, d))
    p = rng.normal(0.0, p_std, size=(K,))
    return mu, vr, p


def _var(vr, floor):
    # softplus through numpy's logaddexp(0, r) = log(1 + e^r): a route independent of the oracle
    return np.logaddexp(0.0, vr) + floor


# ---------------------------------------------------------------- responsibilities

@pytest.mark.parametrize("K,d,floor", [(1, 1, 1e-3), (7, 5, 1e-3), (16, 16, 1e-2), (3, 64, 1e-3)])
def test_log_joint_matches_scipy_logpdf(K, d, floor):
    rng = np.random.default_rng(11 + K + d)
    mu, vr, p = _params(rng, K, d)
    x = rng.normal(size=(40, d))
    got = oracle.log_joint(x, mu, vr, p, floor)
    var = _var(vr, floor)
    logpi = scipy.special.log_softmax(p)
    for k in range(K):
        ref = scipy.stats.multivariate_normal(mean=mu[k], cov=np.diag(var[k])).logpdf(x)
        ref = np.atleast_1d(ref) + logpi[k]
        np.testing.assert_allclose(got[:, k], ref, rtol=1e-10, atol=1e-10)


def test_softplus_extremes_are_stable():
    # var_raw far in both tails: softplus(r) -> r for r >> 0 and -> e^r for r << 0
    K, d, floor = 4, 3, 1e-3
    mu = np.zeros((K, d))
    vr = np.array([[40.0, -40.0, 0.0], [700.0, -700.0, 1.0], [5.0, -5.0, 2.0], [20.0, -20.0, -1.0]])
    p = np.zeros(K)
    x = np.full((1, d), 0.5)
    got = oracle.log_joint(x, mu, vr, p, floor)
    var = _var(vr, floor)
    assert np.all(np.isfinite(got))
    for k in range(K):
        ref = scipy.stats.multivariate_normal(mean=mu[k], cov=np.diag(var[k])).logpdf(x)
        np.testing.assert_allclose(got[0, k], ref + np.log(1.0 / K), rtol=1e-12)


@pytest.mark.parametrize("K,d,floor,seed", [(2, 1, 1e-3, 0), (8, 16, 1e-3, 1), (32, 8, 1e-2, 2),
                                            (128, 64, 1e-3, 3)])
def test_responsibilities_match_sklearn(K, d, floor, seed):
    from sklearn.mixture import GaussianMixture

    rng = np.random.default_rng(seed)
    mu, vr, p = _params(rng, K, d)
    x = rng.normal(size=(200, d))
    var = _var(vr, floor)
    gm = GaussianMixture(n_components=K, covariance_type="diag")
    gm.weights_ = scipy.special.softmax(p)
    gm.means_ = mu
    gm.covariances_ = var
    gm.precisions_cholesky_ = 1.0 / np.sqrt(var)
    ref = gm.predict_proba(x)
    got = oracle.responsibilities(x, mu, vr, p, floor)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_two_component_equal_variance_is_logistic():
    # 1-D, K=2, shared variance s2: p(z=1|x) = sigmoid(w x + b) with
    # w = (m1 - m2)/s2, b = (m2^2 - m1^2)/(2 s2) + log(pi1/pi2)   (linear discriminant)
    m1, m2, r, floor = 0.7, -1.3, 0.2, 1e-3
    s2 = np.logaddexp(0.0, r) + floor
    p = np.array([0.4, -0.9])
    x = np.linspace(-4, 4, 33)[:, None]
    g = oracle.responsibilities(x, np.array([[m1], [m2]]), np.array([[r], [r]]), p, floor)
    logratio = np.log(scipy.special.softmax(p)[0] / scipy.special.softmax(p)[1])
    w = (m1 - m2) / s2
    b = (m2 ** 2 - m1 ** 2) / (2 * s2) + logratio
    np.testing.assert_allclose(g[:, 0], scipy.special.expit(w * x[:, 0] + b), rtol=0, atol=1e-14)
    np.testing.assert_allclose(g.sum(1), 1.0, atol=1e-15)


def test_two_component_unequal_variance_is_quadratic_discriminant():
    # 1-D, K=2: log-odds = log(pi1/pi2) - 0.5 log(s1/s2) - (x-m1)^2/(2 s1) + (x-m2)^2/(2 s2)
    m1, m2, r1, r2, floor = -0.2, 1.1, -0.8, 1.3, 1e-2
    s1 = np.logaddexp(0.0, r1) + floor
    s2 = np.logaddexp(0.0, r2) + floor
    p = np.array([1.2, 0.3])
    x = np.linspace(-3, 3, 25)[:, None]
    g = oracle.responsibilities(x, np.array([[m1], [m2]]), np.array([[r1], [r2]]), p, floor)
    lo = (p[0] - p[1]) - 0.5 * np.log(s1 / s2) - (x[:, 0] - m1) ** 2 / (2 * s1) \
        + (x[:, 0] - m2) ** 2 / (2 * s2)
    np.testing.assert_allclose(g[:, 0], scipy.special.expit(lo), rtol=0, atol=1e-14)


def test_identical_components_give_prior():
    rng = np.random.default_rng(5)
    K, d = 6, 4
    mu = np.tile(rng.normal(size=(1, d)), (K, 1))
    vr = np.tile(rng.normal(size=(1, d)), (K, 1))
    p = rng.normal(size=K)
    x = rng.normal(size=(17, d))
    g = oracle.responsibilities(x, mu, vr, p, 1e-3)
    np.testing.assert_allclose(g, np.tile(scipy.special.softmax(p), (17, 1)), atol=1e-15)


def test_prior_logit_shift_invariance():
    rng = np.random.default_rng(6)
    mu, vr, p = _params(rng, 9, 5)
    x = rng.normal(size=(30, 5))
    g1 = oracle.responsibilities(x, mu, vr, p, 1e-3)
    g2 = oracle.responsibilities(x, mu, vr, p + 3.75, 1e-3)
    np.testing.assert_allclose(g1, g2, atol=1e-14)


# ---------------------------------------------------------------- mixing

def _brute(gq, gk, v, eps, causal):
    """Independent N x N brute force: materialise A = Gamma_Q Gamma_K^T (lower-triangular
    incl. the diagonal when causal) and row-normalise A [V, 1]."""
    A = gq @ gk.T
    if causal:
        A = np.tril(A)
    return (A @ v) / (A.sum(axis=1, keepdims=True) + eps)


def _random_problem(rng, B, H, N, dr, dv, K, mu_std=1.0, x_std=1.0):
    qr = rng.normal(0, x_std, size=(B, H, N, dr))
    kr = rng.normal(0, x_std, size=(B, H, N, dr))
    v = rng.normal(size=(B, H, N, dv))
    mu = rng.normal(0, mu_std, size=(H, K, dr))
    vr = rng.normal(0, 0.5, size=(H, K, dr))
    p = rng.normal(size=(H, K))
    return qr, kr, v, mu, vr, p


@settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(N=st.integers(1, 96), K=st.integers(1, 24), dr=st.integers(1, 12), dv=st.integers(1, 12),
       causal=st.booleans(), seed=st.integers(0, 2 ** 31 - 1),
       eps=st.sampled_from([1e-6, 1e-3, 0.5]))
def test_forward_matches_bruteforce(N, K, dr, dv, causal, seed, eps):
    rng = np.random.default_rng(seed)
    qr, kr, v, mu, vr, p = _random_problem(rng, 1, 2, N, dr, dv, K)
    out, gq, gk = oracle.forward(qr, kr, v, mu, vr, p, causal, eps, 1e-3, return_gamma=True)
    for h in range(2):
        ref = _brute(gq[0, h], gk[0, h], v[0, h], eps, causal)
        assert metrics.rowrel(out[0, h][None, None], ref[None, None]) < 1e-12


def test_forward_gamma_matches_sklearn_path():
    # the Gamma returned by the full forward is the same posterior sklearn computes
    from sklearn.mixture import GaussianMixture

    rng = np.random.default_rng(9)
    qr, kr, v, mu, vr, p = _random_problem(rng, 2, 3, 50, 6, 5, 10)
    _, gq, gk = oracle.forward(qr, kr, v, mu, vr, p, False, 1e-6, 1e-3, return_gamma=True)
    for h in range(3):
        var = _var(vr[h], 1e-3)
        gm = GaussianMixture(n_components=10, covariance_type="diag")
        gm.weights_, gm.means_, gm.covariances_ = scipy.special.softmax(p[h]), mu[h], var
        gm.precisions_cholesky_ = 1.0 / np.sqrt(var)
        for b in range(2):
            np.testing.assert_allclose(gq[b, h], gm.predict_proba(qr[b, h]), atol=1e-12)
            np.testing.assert_allclose(gk[b, h], gm.predict_proba(kr[b, h]), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_single_component_is_mean_or_prefix_mean(causal):
    rng = np.random.default_rng(3)
    N, eps = 37, 1e-3
    qr, kr, v, mu, vr, p = _random_problem(rng, 1, 1, N, 4, 6, 1)
    out = oracle.forward(qr, kr, v, mu, vr, p, causal, eps, 1e-3)[0, 0]
    vv = v[0, 0]
    if causal:
        ref = np.cumsum(vv, axis=0) / (np.arange(1, N + 1)[:, None] + eps)
    else:
        ref = np.tile(vv.sum(0) / (N + eps), (N, 1))
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_components_closed_form(causal):
    # gamma = pi for every token: A_ij = |pi|^2, so O_i = sum v / (n_i + eps/|pi|^2)
    rng = np.random.default_rng(4)
    N, K, d, eps = 23, 5, 3, 0.01
    qr, kr, v, mu, vr, p = _random_problem(rng, 1, 1, N, d, 4, K)
    mu[0] = mu[0, :1]
    vr[0] = vr[0, :1]
    out = oracle.forward(qr, kr, v, mu, vr, p, causal, eps, 1e-3)[0, 0]
    pi2 = float((scipy.special.softmax(p[0]) ** 2).sum())
    vv = v[0, 0]
    if causal:
        ref = np.cumsum(vv, axis=0) / (np.arange(1, N + 1)[:, None] + eps / pi2)
    else:
        ref = np.tile(vv.sum(0) / (N + eps / pi2), (N, 1))
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-15)


def test_affinity_rank_at_most_K_and_semiseparable():
    rng = np.random.default_rng(8)
    N, K = 120, 7
    qr, kr, v, mu, vr, p = _random_problem(rng, 1, 1, N, 5, 3, K)
    _, gq, gk = oracle.forward(qr, kr, v, mu, vr, p, True, 1e-6, 1e-3, return_gamma=True)
    A = gq[0, 0] @ gk[0, 0].T
    s = np.linalg.svd(A, compute_uv=False)
    assert s[K] <= 1e-10 * s[0]
    assert np.all(A >= 0)
    # any block strictly below the diagonal of tril(A) is a block of A: rank <= K
    L = np.tril(A)
    for split in (20, 60, 100):
        blk = L[split:, :split]
        sb = np.linalg.svd(blk, compute_uv=False)
        assert len(sb) <= K or sb[K] <= 1e-10 * sb[0]


def test_responsibility_rows_on_simplex():
    rng = np.random.default_rng(12)
    qr, kr, v, mu, vr, p = _random_problem(rng, 2, 2, 64, 8, 4, 33, mu_std=2.0)
    _, gq, gk = oracle.forward(qr, kr, v, mu, vr, p, False, 1e-6, 1e-3, return_gamma=True)
    for g in (gq, gk):
        assert np.all(g >= 0)
        np.testing.assert_allclose(g.sum(-1), 1.0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_output_bounded_linear_and_equivariant(causal):
    rng = np.random.default_rng(13)
    N = 48
    qr, kr, v, mu, vr, p = _random_problem(rng, 1, 1, N, 6, 5, 9)
    o1 = oracle.forward(qr, kr, v, mu, vr, p, causal, 1e-6, 1e-3)
    # convex combination scaled by A1/(A1+eps) < 1
    assert np.all(np.abs(o1) <= np.abs(v).max(axis=2, keepdims=True) + 1e-12)
    # linear in V
    v2 = rng.normal(size=v.shape)
    o2 = oracle.forward(qr, kr, v2, mu, vr, p, causal, 1e-6, 1e-3)
    o12 = oracle.forward(qr, kr, 2.0 * v - 3.0 * v2, mu, vr, p, causal, 1e-6, 1e-3)
    np.testing.assert_allclose(o12, 2.0 * o1 - 3.0 * o2, atol=1e-12)
    if not causal:
        # permuting keys with their values changes nothing; permuting queries permutes rows
        perm = rng.permutation(N)
        o3 = oracle.forward(qr[:, :, perm], kr[:, :, perm], v[:, :, perm], mu, vr, p, False,
                            1e-6, 1e-3)
        np.testing.assert_allclose(o3, o1[:, :, perm], atol=1e-13)


def test_causal_outputs_ignore_the_future_exactly():
    rng = np.random.default_rng(14)
    N, cut = 40, 17
    qr, kr, v, mu, vr, p = _random_problem(rng, 1, 2, N, 4, 3, 6)
    o1 = oracle.forward(qr, kr, v, mu, vr, p, True, 1e-6, 1e-3)
    qr2, kr2, v2 = qr.copy(), kr.copy(), v.copy()
    qr2[:, :, cut + 1:] = rng.normal(size=qr2[:, :, cut + 1:].shape)
    kr2[:, :, cut + 1:] = rng.normal(size=kr2[:, :, cut + 1:].shape)
    v2[:, :, cut + 1:] = 100 * rng.normal(size=v2[:, :, cut + 1:].shape)
    o2 = oracle.forward(qr2, kr2, v2, mu, vr, p, True, 1e-6, 1e-3)
    assert np.array_equal(o1[:, :, :cut + 1], o2[:, :, :cut + 1])
    assert not np.allclose(o1[:, :, cut + 1:], o2[:, :, cut + 1:])
    # and the last position of the causal variant equals the bidirectional row
    ob = oracle.forward(qr, kr, v, mu, vr, p, False, 1e-6, 1e-3)
    np.testing.assert_allclose(o1[:, :, -1], ob[:, :, -1], atol=1e-13)


def test_empty_sequence():
    rng = np.random.default_rng(15)
    qr, kr, v, mu, vr, p = _random_problem(rng, 1, 1, 0, 4, 3, 5)
    for causal in (False, True):
        out = oracle.forward(qr, kr, v, mu, vr, p, causal, 1e-6, 1e-3)
        assert out.shape == (1, 1, 0, 3)


# ---------------------------------------------------------------- cross variant
# German page, closing paragraph: cross-attention named as future work.  Reading: the
# bidirectional write/read with the memory over Nk key rows and the read over Nq query rows.

def _cross_problem(rng, B, H, Nq, Nk, dr, dv, K):
    qr = rng.normal(size=(B, H, Nq, dr))
    kr = rng.normal(size=(B, H, Nk, dr))
    v = rng.normal(size=(B, H, Nk, dv))
    mu = rng.normal(size=(H, K, dr))
    vr = rng.normal(0, 0.5, size=(H, K, dr))
    p = rng.normal(size=(H, K))
    return qr, kr, v, mu, vr, p


@settings(max_examples=20, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(Nq=st.integers(1, 64), Nk=st.integers(1, 96), K=st.integers(1, 16), dr=st.integers(1, 8),
       dv=st.integers(1, 8), seed=st.integers(0, 2 ** 31 - 1), eps=st.sampled_from([1e-6, 0.5]))
def test_cross_matches_bruteforce(Nq, Nk, K, dr, dv, seed, eps):
    # Nq x Nk affinity A = Gamma_Q Gamma_K^T, row-normalised A [V, 1]; Gamma from sklearn's
    # posterior, not from the oracle
    from sklearn.mixture import GaussianMixture

    rng = np.random.default_rng(seed)
    qr, kr, v, mu, vr, p = _cross_problem(rng, 1, 2, Nq, Nk, dr, dv, K)
    out = oracle.forward_cross(qr, kr, v, mu, vr, p, eps, 1e-3)
    assert out.shape == (1, 2, Nq, dv)
    for h in range(2):
        var = _var(vr[h], 1e-3)
        gm = GaussianMixture(n_components=K, covariance_type="diag")
        gm.weights_, gm.means_, gm.covariances_ = scipy.special.softmax(p[h]), mu[h], var
        gm.precisions_cholesky_ = 1.0 / np.sqrt(var)
        ref = _brute(gm.predict_proba(qr[0, h]), gm.predict_proba(kr[0, h]), v[0, h], eps, False)
        assert metrics.rowrel(out[0, h][None, None], ref[None, None]) < 1e-10


def test_cross_closed_forms():
    rng = np.random.default_rng(21)
    Nq, Nk, eps = 13, 41, 1e-3
    # K = 1: every query reads the mean of the Nk values
    qr, kr, v, mu, vr, p = _cross_problem(rng, 1, 1, Nq, Nk, 4, 5, 1)
    out = oracle.forward_cross(qr, kr, v, mu, vr, p, eps, 1e-3)[0, 0]
    np.testing.assert_allclose(out, np.tile(v[0, 0].sum(0) / (Nk + eps), (Nq, 1)), rtol=1e-13)
    # identical components: gamma = pi, A_ij = |pi|^2
    qr, kr, v, mu, vr, p = _cross_problem(rng, 1, 1, Nq, Nk, 3, 4, 6)
    mu[0] = mu[0, :1]
    vr[0] = vr[0, :1]
    out = oracle.forward_cross(qr, kr, v, mu, vr, p, 0.01, 1e-3)[0, 0]
    pi2 = float((scipy.special.softmax(p[0]) ** 2).sum())
    np.testing.assert_allclose(out, np.tile(v[0, 0].sum(0) / (Nk + 0.01 / pi2), (Nq, 1)), rtol=1e-13)
    # empty memory: 0 / (0 + eps); no queries: empty output
    qr, kr, v, mu, vr, p = _cross_problem(rng, 1, 1, Nq, 0, 3, 4, 6)
    assert np.array_equal(oracle.forward_cross(qr, kr, v, mu, vr, p, 0.5, 1e-3), np.zeros((1, 1, Nq, 4)))
    qr, kr, v, mu, vr, p = _cross_problem(rng, 1, 1, 0, 9, 3, 4, 6)
    assert oracle.forward_cross(qr, kr, v, mu, vr, p, 0.5, 1e-3).shape == (1, 1, 0, 4)


def test_cross_invariants():
    rng = np.random.default_rng(22)
    Nq, Nk = 19, 57
    qr, kr, v, mu, vr, p = _cross_problem(rng, 2, 2, Nq, Nk, 6, 5, 9)
    o1 = oracle.forward_cross(qr, kr, v, mu, vr, p, 1e-6, 1e-3)
    # permuting keys with their values changes nothing; permuting queries permutes rows
    pk, pq = rng.permutation(Nk), rng.permutation(Nq)
    o2 = oracle.forward_cross(qr[:, :, pq], kr[:, :, pk], v[:, :, pk], mu, vr, p, 1e-6, 1e-3)
    np.testing.assert_allclose(o2, o1[:, :, pq], atol=1e-13)
    # each query row depends on its own routing vector only: a query reads the same row
    # whatever the other queries are
    o3 = oracle.forward_cross(qr[:, :, :5], kr, v, mu, vr, p, 1e-6, 1e-3)
    np.testing.assert_allclose(o3, o1[:, :, :5], atol=1e-15)
    # convex combination of the values, scaled by A1/(A1+eps) < 1
    assert np.all(np.abs(o1) <= np.abs(v).max(axis=2, keepdims=True) + 1e-12)
    # with the same rows for queries and keys it is the bidirectional self-mixing
    qr, kr, v, mu, vr, p = _cross_problem(rng, 1, 2, 30, 30, 4, 3, 5)
    np.testing.assert_allclose(oracle.forward_cross(qr, kr, v, mu, vr, p, 1e-3, 1e-3),
                               oracle.forward(qr, kr, v, mu, vr, p, False, 1e-3, 1e-3), rtol=0, atol=0)


# ---------------------------------------------------------------- decode step
# Core mechanism item 3 read as a recurrence: the causal memory after positions 0..t-1 is
# [S | z]; a step adds gamma_K,t (x) [v_t | 1] and reads row t.

def _sk_gamma(x, mu, vr, p, floor=1e-3):
    from sklearn.mixture import GaussianMixture
    var = _var(vr, floor)
    gm = GaussianMixture(n_components=mu.shape[0], covariance_type="diag")
    gm.weights_, gm.means_, gm.covariances_ = scipy.special.softmax(p), mu, var
    gm.precisions_cholesky_ = 1.0 / np.sqrt(var)
    return gm.predict_proba(x)


@pytest.mark.parametrize("N,K,dr,dv,split", [(1, 1, 3, 2, 0), (25, 7, 5, 4, 0), (40, 16, 8, 6, 17),
                                             (64, 33, 4, 9, 63)])
def test_memory_then_decode_matches_causal_bruteforce(N, K, dr, dv, split):
    rng = np.random.default_rng(31 + N + K)
    qr, kr, v, mu, vr, p = _random_problem(rng, 1, 2, N, dr, dv, K)
    eps = 1e-3
    # prefill: the memory of positions 0..split-1, against an sklearn-posterior reference
    state = oracle.memory(kr[:, :, :split], v[:, :, :split], mu, vr, p, 1e-3)
    for h in range(2):
        gk = _sk_gamma(kr[0, h, :split], mu[h], vr[h], p[h]) if split else np.zeros((0, K))
        ref = np.concatenate([gk.T @ v[0, h, :split], gk.sum(0)[:, None]], axis=1)
        np.testing.assert_allclose(state[0, h], ref, rtol=1e-12, atol=1e-13)
    # decode the remaining positions one at a time: row t of the causal brute force
    outs = []
    for t in range(split, N):
        outs.append(oracle.decode_step(qr[:, :, t], kr[:, :, t], v[:, :, t], mu, vr, p, state, eps, 1e-3))
    got = np.stack(outs, axis=2) if outs else np.zeros((1, 2, 0, dv))
    for h in range(2):
        gq = _sk_gamma(qr[0, h], mu[h], vr[h], p[h])
        gk = _sk_gamma(kr[0, h], mu[h], vr[h], p[h])
        ref = _brute(gq, gk, v[0, h], eps, True)[split:]
        assert metrics.rowrel(got[0, h][None, None], ref[None, None]) < 1e-10
    # the state after the last step is the memory of the whole sequence
    np.testing.assert_allclose(state, oracle.memory(kr, v, mu, vr, p, 1e-3), rtol=1e-12, atol=1e-13)


def test_decode_closed_forms():
    rng = np.random.default_rng(41)
    # K = 1: gamma = 1, the step returns the running mean of v (prefix mean)
    qr, kr, v, mu, vr, p = _random_problem(rng, 1, 1, 12, 3, 4, 1)
    state = np.zeros((1, 1, 1, 5))
    for t in range(12):
        o = oracle.decode_step(qr[:, :, t], kr[:, :, t], v[:, :, t], mu, vr, p, state, 1e-6, 1e-3)
        np.testing.assert_allclose(o[0, 0], v[0, 0, :t + 1].sum(0) / (t + 1 + 1e-6), rtol=1e-13)
    # a single token into an empty memory: O = (gq.gk) v / (gq.gk + eps)
    qr, kr, v, mu, vr, p = _random_problem(rng, 1, 1, 1, 5, 3, 6)
    state = np.zeros((1, 1, 6, 4))
    o = oracle.decode_step(qr[:, :, 0], kr[:, :, 0], v[:, :, 0], mu, vr, p, state, 0.25, 1e-3)
    a = float(_sk_gamma(qr[0, 0, :1], mu[0], vr[0], p[0])[0] @ _sk_gamma(kr[0, 0, :1], mu[0], vr[0], p[0])[0])
    np.testing.assert_allclose(o[0, 0], a * v[0, 0, 0] / (a + 0.25), rtol=1e-12)
    # the memory of an empty prefix is zero
    assert not oracle.memory(kr[:, :, :0], v[:, :, :0], mu, vr, p, 1e-3).any()


# ---------------------------------------------------------------- responsibility statistics
# The pages' interpretability analysis (components used, usage entropy, hard assignments):
# hard = argmax of the posterior (lowest index on ties), counts = its histogram per head
# over (b, n), usage = sum of the posteriors, used = #{counts > 0}, entropy = Shannon
# entropy of counts / (B N) over ln K.

@pytest.mark.parametrize("B,H,N,dr,K", [(2, 3, 50, 5, 7), (1, 2, 1, 3, 4), (3, 1, 33, 8, 16)])
def test_resp_stats_match_sklearn(B, H, N, dr, K):
    rng = np.random.default_rng(71 + N + K)
    x, _, _, mu, vr, p = _random_problem(rng, B, H, N, dr, 1, K, mu_std=1.5)
    r = oracle.resp_stats(x, mu, vr, p, 1e-3)
    for h in range(H):
        gam = np.concatenate([_sk_gamma(x[b, h], mu[h], vr[h], p[h]) for b in range(B)])
        from sklearn.mixture import GaussianMixture
        gm = GaussianMixture(n_components=K, covariance_type="diag")
        var = _var(vr[h], 1e-3)
        gm.weights_, gm.means_, gm.covariances_ = scipy.special.softmax(p[h]), mu[h], var
        gm.precisions_cholesky_ = 1.0 / np.sqrt(var)
        pred = np.concatenate([gm.predict(x[b, h]) for b in range(B)])
        np.testing.assert_array_equal(r["hard"][:, h].reshape(-1), pred)
        cnt = np.bincount(pred, minlength=K)
        np.testing.assert_array_equal(r["counts"][h], cnt)
        np.testing.assert_allclose(r["usage"][h], gam.sum(0), rtol=1e-12, atol=1e-12)
        assert r["used"][h] == np.count_nonzero(cnt)
        ref_ent = scipy.stats.entropy(cnt) / np.log(K) if K > 1 else 0.0
        np.testing.assert_allclose(r["entropy"][h], ref_ent, rtol=1e-12, atol=1e-15)
    # soft usage sums to the number of rows; counts too
    np.testing.assert_allclose(r["usage"].sum(1), B * N, rtol=1e-12)
    np.testing.assert_array_equal(r["counts"].sum(1), B * N)


def test_resp_stats_closed_forms():
    rng = np.random.default_rng(72)
    # K = 1: everything to component 0, entropy 0
    x, _, _, mu, vr, p = _random_problem(rng, 2, 2, 9, 3, 1, 1)
    r = oracle.resp_stats(x, mu, vr, p, 1e-3)
    assert (r["hard"] == 0).all() and (r["counts"] == 18).all() and (r["used"] == 1).all()
    np.testing.assert_allclose(r["usage"], 18.0, rtol=1e-14)
    assert (r["entropy"] == 0.0).all()
    # identical Gaussians, different priors: gamma = pi for every row, hard = argmax prior
    K, dr = 5, 4
    mu = np.tile(rng.normal(size=(1, 1, dr)), (1, K, 1))
    vr = np.tile(rng.normal(size=(1, 1, dr)), (1, K, 1))
    p = np.array([[0.1, 0.7, -0.3, 0.7, 0.2]])
    x = rng.normal(size=(2, 1, 6, dr))
    r = oracle.resp_stats(x, mu, vr, p, 1e-3)
    assert (r["hard"] == 1).all()  # components 1 and 3 tie on the prior: the lower index
    np.testing.assert_allclose(r["usage"][0], 12 * scipy.special.softmax(p[0]), rtol=1e-12)
    assert r["used"][0] == 1 and r["entropy"][0] == 0.0
    # each row at a distinct, well-separated mean, every component hit equally often:
    # uniform usage, entropy exactly 1
    K, dr = 8, 3
    mu = 10.0 * rng.normal(size=(1, K, dr))
    vr = np.full((1, K, dr), -4.0)
    p = np.zeros((1, K))
    x = np.stack([mu[0][np.arange(4 * K) % K]]).reshape(1, 1, 4 * K, dr)
    r = oracle.resp_stats(x, mu, vr, p, 1e-3)
    np.testing.assert_array_equal(r["hard"][0, 0], np.arange(4 * K) % K)
    assert (r["counts"][0] == 4).all() and r["used"][0] == K
    np.testing.assert_allclose(r["entropy"][0], 1.0, rtol=1e-14)
    # two of the components take all rows equally: entropy ln 2 / ln K
    x2 = np.stack([mu[0][np.arange(6) % 2]]).reshape(1, 1, 6, dr)
    r = oracle.resp_stats(x2, mu, vr, p, 1e-3)
    assert r["used"][0] == 2
    np.testing.assert_allclose(r["entropy"][0], np.log(2) / np.log(K), rtol=1e-14)
    # no rows: nothing counted
    r = oracle.resp_stats(x[:, :, :0], mu, vr, p, 1e-3)
    assert r["counts"].sum() == 0 and r["used"][0] == 0 and r["entropy"][0] == 0.0


# ---------------------------------------------------------------- backward
# The pages train the mixture end to end by backpropagation.  The oracle's hand-written chain
# rule is pinned by central differences of the oracle forward, by autograd through an fp64
# torch formulation of the forward written here from the definitions, and by invariants.

def _loss(qr, kr, v, mu, vr, p, dout, causal, eps):
    return float((oracle.forward(qr, kr, v, mu, vr, p, causal, eps, 1e-3) * dout).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_central_differences(causal):
    rng = np.random.default_rng(101 + causal)
    B, H, N, dr, dv, K = 2, 2, 5, 3, 2, 4
    qr, kr, v, mu, vr, p = _random_problem(rng, B, H, N, dr, dv, K)
    dout = rng.normal(size=(B, H, N, dv))
    eps = 0.05
    g = oracle.backward(qr, kr, v, mu, vr, p, dout, causal, eps, 1e-3)
    args = {"qr": qr, "kr": kr, "v": v, "mu": mu, "vr": vr, "p": p}
    names = {"qr": "dqr", "kr": "dkr", "v": "dv", "mu": "dmu", "vr": "dvar_raw", "p": "dprior"}
    step = 1e-5
    for a, arr in args.items():
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + step
            lp = _loss(args["qr"], args["kr"], args["v"], args["mu"], args["vr"], args["p"], dout, causal, eps)
            arr[idx] = old - step
            lm = _loss(args["qr"], args["kr"], args["v"], args["mu"], args["vr"], args["p"], dout, causal, eps)
            arr[idx] = old
            fd[idx] = (lp - lm) / (2 * step)
        np.testing.assert_allclose(g[names[a]], fd, rtol=1e-6, atol=1e-8, err_msg=a)


def _torch_forward(qr, kr, v, mu, vr, p, causal, eps, floor):
    import torch
    var = torch.nn.functional.softplus(vr) + floor                      # [H,K,d]
    logpi = p - torch.logsumexp(p, dim=-1, keepdim=True)                 # [H,K]

    def post(x):                                                         # x [B,H,N,d]
        diff = x[:, :, :, None, :] - mu[None, :, None, :, :]             # [B,H,N,K,d]
        logn = -0.5 * (np.log(2 * np.pi) + torch.log(var)[None, :, None] + diff ** 2 / var[None, :, None]).sum(-1)
        return torch.softmax(logpi[None, :, None, :] + logn, dim=-1)     # [B,H,N,K]

    gq, gk = post(qr), post(kr)
    aff = gq @ gk.transpose(-1, -2)                                      # [B,H,N,N]
    if causal:
        aff = torch.tril(aff)
    num = aff @ v
    den = aff.sum(-1, keepdim=True) + eps
    return num / den


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N,dr,dv,K", [(2, 3, 17, 5, 4, 6), (1, 2, 33, 8, 3, 16), (1, 1, 1, 2, 2, 1)])
def test_backward_matches_autograd(B, H, N, dr, dv, K, causal):
    import torch
    rng = np.random.default_rng(111 + N + K + causal)
    qr, kr, v, mu, vr, p = _random_problem(rng, B, H, N, dr, dv, K)
    dout = rng.normal(size=(B, H, N, dv))
    eps = 1e-3
    ts = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (qr, kr, v, mu, vr, p)]
    out = _torch_forward(*ts, causal, eps, 1e-3)
    (out * torch.tensor(dout)).sum().backward()
    g = oracle.backward(qr, kr, v, mu, vr, p, dout, causal, eps, 1e-3)
    for t, name in zip(ts, ("dqr", "dkr", "dv", "dmu", "dvar_raw", "dprior")):
        ref = t.grad.numpy()
        np.testing.assert_allclose(g[name], ref, rtol=1e-9, atol=1e-11 * max(1.0, np.abs(ref).max()), err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    rng = np.random.default_rng(121 + causal)
    B, H, N, dr, dv, K = 2, 2, 40, 4, 3, 7
    qr, kr, v, mu, vr, p = _random_problem(rng, B, H, N, dr, dv, K)
    dout = rng.normal(size=(B, H, N, dv))
    eps = 1e-3
    g = oracle.backward(qr, kr, v, mu, vr, p, dout, causal, eps, 1e-3)
    L = _loss(qr, kr, v, mu, vr, p, dout, causal, eps)
    # prior logits: the forward is invariant to a common shift, so the gradient sums to zero
    np.testing.assert_allclose(g["dprior"].sum(-1), 0.0, atol=1e-12)
    # the output is linear in V: sum dV * V = L
    np.testing.assert_allclose((g["dv"] * v).sum(), L, rtol=1e-12)
    # shifting every routing row and every mean of a head by one vector changes nothing
    tot = g["dqr"].sum(axis=(0, 2)) + g["dkr"].sum(axis=(0, 2)) + g["dmu"].sum(axis=1)
    np.testing.assert_allclose(tot, 0.0, atol=1e-10)
    if causal:
        # rows at or after t receive gradient only from outputs at or after them: with dO = 0
        # from t on, dv and dk vanish there, and dq too
        t = 25
        d2 = dout.copy()
        d2[:, :, t:] = 0.0
        g2 = oracle.backward(qr, kr, v, mu, vr, p, d2, causal, eps, 1e-3)
        assert not g2["dv"][:, :, t:].any() and not g2["dkr"][:, :, t:].any() and not g2["dqr"][:, :, t:].any()
        # and the gradients before t equal those of the prefix problem alone
        gp = oracle.backward(qr[:, :, :t], kr[:, :, :t], v[:, :, :t], mu, vr, p, dout[:, :, :t], causal, eps, 1e-3)
        for name in ("dqr", "dkr", "dv"):
            np.testing.assert_allclose(g2[name][:, :, :t], gp[name], rtol=1e-12, atol=1e-14)
        for name in ("dmu", "dvar_raw", "dprior"):
            np.testing.assert_allclose(g2[name], gp[name], rtol=1e-10, atol=1e-13)


def test_golden_fixture_regression():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_gma.json")
    fx = json.load(open(path))
    inp = {k: np.asarray(v) for k, v in fx["inputs"].items()}
    for key, causal in (("bidirectional", False), ("causal", True)):
        out, gq, gk = oracle.forward(inp["qr"], inp["kr"], inp["v"], inp["mu"], inp["var_raw"],
                                     inp["prior_logits"], causal, fx["eps"], fx["var_floor"],
                                     return_gamma=True)
        np.testing.assert_allclose(out, np.asarray(fx[key]["out"]), rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(gq, np.asarray(fx[key]["gamma_q"]), rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(gk, np.asarray(fx[key]["gamma_k"]), rtol=1e-14, atol=1e-15)
