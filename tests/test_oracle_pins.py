"""Pins for the fp64 oracle against what the pages and the mathematics fix.

Each test names the property it checks and the passage (page title plus
section) or the mathematical fact behind it.  A plausible mistake in the
oracle -- a dropped norm term, a wrong sign, a missing 1/sqrt(m), a
transposed operand, an unorthogonalised block, a wrong mask -- fails at least
one of them.  None of these tests re-types the oracle's formula: each compares
it with an independent fact (closed form, invariant, brute force, library
routine, distribution law).
"""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle

pytestmark = []


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# The random stream (pages name none; the draw must be uniform / Gaussian).
# ---------------------------------------------------------------------------
def test_uniforms_are_uniform_and_in_half_open_interval():
    u = oracle.uniforms(123, 0, 200_000)
    assert u.min() > 0.0 and u.max() <= 1.0
    assert scipy.stats.kstest(u, "uniform").pvalue > 1e-3
    # consecutive draws uncorrelated
    assert abs(np.corrcoef(u[:-1], u[1:])[0, 1]) < 5 / math.sqrt(u.size)


def test_uniform_stream_is_counter_based():
    # any window of the stream equals the same slice of a longer draw
    a = oracle.uniforms(9, 0, 1000)
    b = oracle.uniforms(9, 517, 100)
    np.testing.assert_array_equal(a[517:617], b)
    # different seeds give different streams
    assert not np.array_equal(oracle.uniforms(10, 0, 100), a[:100])


def test_normals_are_standard_normal():
    z = oracle.normals(77, 0, 200_000)
    assert scipy.stats.kstest(z, "norm").pvalue > 1e-3
    assert abs(z.mean()) < 5 / math.sqrt(z.size)
    assert abs(z.var() - 1.0) < 5 * math.sqrt(2.0 / z.size)
    # the cosine and sine halves of each Box-Muller pair are uncorrelated
    assert abs(np.corrcoef(z[0::2], z[1::2])[0, 1]) < 5 / math.sqrt(z.size / 2)


def test_normals_window_consistency_odd_start():
    full = oracle.normals(5, 0, 101)
    np.testing.assert_array_equal(oracle.normals(5, 37, 20), full[37:57])
    np.testing.assert_array_equal(oracle.normals(5, 38, 1), full[38:39])


# ---------------------------------------------------------------------------
# P1-P3: the projection W (summary page, "Key contributions" and
# "Limitations": positive orthogonal random features, orthogonal for at most
# d rows; block reading with chi(d) norms).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("m,d", [(16, 16), (256, 64), (512, 128), (40, 16)])
def test_P1_block_orthogonality(m, d):
    W = oracle.draw_w(1000 + m + d, m, d)
    assert W.shape == (m, d)
    for b0 in range(0, m, d):
        Wb = W[b0:b0 + d]
        G = Wb @ Wb.T
        diag = np.diag(G)
        off = G - np.diag(diag)
        assert np.max(np.abs(off)) <= 1e-12 * diag.mean()
    # fp32-stored W keeps orthogonality to fp32 rounding
    W32 = W.astype(np.float32).astype(np.float64)
    for b0 in range(0, m, d):
        Wb = W32[b0:b0 + d]
        G = Wb @ Wb.T
        off = G - np.diag(np.diag(G))
        assert np.max(np.abs(off)) <= 1e-6 * np.diag(G).mean()


def test_P1_blocks_are_not_orthogonal_to_each_other():
    # independent blocks: cross-block products are O(|w|^2 / sqrt(d)), not zero
    W = oracle.draw_w(3, 128, 64)
    cross = W[:64] @ W[64:].T
    assert np.max(np.abs(cross)) > 1.0


@pytest.mark.parametrize("d", [16, 64])
def test_P2_row_norms_follow_chi_d(d):
    W = oracle.draw_w(2024 + d, 256 * d if d == 16 else 64 * d, d)
    s = np.linalg.norm(W, axis=1)
    n = s.size
    assert abs(np.mean(s ** 2) - d) < 5 * math.sqrt(2 * d / n)
    assert scipy.stats.kstest(s, scipy.stats.chi(d).cdf).pvalue > 1e-3
    # norms are independent of the direction: the norm is uncorrelated with
    # the first coordinate of the unit direction
    u = W / s[:, None]
    assert abs(np.corrcoef(s, u[:, 0])[0, 1]) < 5 / math.sqrt(n)


def test_P3_rows_are_marginally_standard_normal():
    d = 16
    W = oracle.draw_w(99, 16 * 4000, d)
    n = W.shape[0]
    mean = W.mean(axis=0)
    assert np.max(np.abs(mean)) < 5 / math.sqrt(n)
    C = np.cov(W.T)
    assert np.max(np.abs(np.diag(C) - 1)) < 5 * math.sqrt(2.0 / n)
    off = C - np.diag(np.diag(C))
    assert np.max(np.abs(off)) < 5 / math.sqrt(n)
    # each coordinate is N(0,1)
    assert scipy.stats.kstest(W[:, 3], "norm").pvalue > 1e-3


def test_draw_w_partial_last_block():
    # m not a multiple of d: the last block takes its first (m mod d) rows
    Wfull = oracle.draw_w(11, 32, 16)
    W = oracle.draw_w(11, 24, 16)
    np.testing.assert_array_equal(W[:16], Wfull[:16])
    Wb = W[16:]
    G = Wb @ Wb.T
    assert np.max(np.abs(G - np.diag(np.diag(G)))) <= 1e-12 * np.diag(G).mean()


# ---------------------------------------------------------------------------
# P4, P5: closed forms of the feature map that hold for every W.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("m,d", [(16, 16), (256, 64), (37, 8)])
def test_P4_phi_x_dot_phi_minus_x(m, d):
    rng = _rng(m * d)
    W = rng.standard_normal((m, d)) * 1.3
    X = rng.standard_normal((50, d)) * 0.6
    lhs = np.sum(oracle.phi(X, W) * oracle.phi(-X, W), axis=1)
    rhs = np.exp(-np.sum(X * X, axis=1))
    np.testing.assert_allclose(lhs, rhs, rtol=1e-13, atol=0)


def test_P4_phi_scales_with_one_over_sqrt_m():
    # duplicating every row of W doubles m and leaves phi^T phi unchanged
    rng = _rng(5)
    W = rng.standard_normal((16, 8))
    X = rng.standard_normal((4, 8)) * 0.5
    Y = rng.standard_normal((4, 8)) * 0.5
    a = oracle.phi(X, W) @ oracle.phi(Y, W).T
    W2 = np.concatenate([W, W])
    b = oracle.phi(X, W2) @ oracle.phi(Y, W2).T
    np.testing.assert_allclose(a, b, rtol=1e-14)


@pytest.mark.parametrize("m", [1, 16, 256])
def test_P5_phi_of_zero(m):
    W = _rng(m).standard_normal((m, 8))
    np.testing.assert_allclose(oracle.phi(np.zeros((1, 8)), W), 1 / math.sqrt(m), rtol=1e-15)


def test_phi_is_positive_and_matches_single_feature_closed_form():
    # one feature, one coordinate: phi = exp(w x - x^2/2)
    W = np.array([[1.5]])
    x = np.array([[0.4]])
    np.testing.assert_allclose(oracle.phi(x, W), [[math.exp(1.5 * 0.4 - 0.08)]], rtol=1e-15)
    X = _rng(1).standard_normal((100, 16)) * 3
    assert np.all(oracle.phi(X, _rng(2).standard_normal((64, 16))) > 0)


# ---------------------------------------------------------------------------
# P6, P7: unbiasedness and lower variance ("Rethinking Attention with
# Performers", abstract; summary page "Key contributions").
# ---------------------------------------------------------------------------
def _pair(norm2, seed, d=16):
    rng = _rng(seed)
    x = rng.standard_normal(d)
    y = rng.standard_normal(d)
    s = x + y
    f = math.sqrt(norm2) / np.linalg.norm(s)
    return x * f, y * f


def _block_estimates(W, x, y, d):
    # each d-row block is one independent estimator with m = d features
    nb = W.shape[0] // d
    px = oracle.phi(x[None, :], W)[0].reshape(nb, d) * math.sqrt(W.shape[0] / d)
    py = oracle.phi(y[None, :], W)[0].reshape(nb, d) * math.sqrt(W.shape[0] / d)
    return np.sum(px * py, axis=1)


@pytest.mark.slow
@pytest.mark.parametrize("norm2", [0.25, 1.0])
def test_P6_unbiased_softmax_kernel(norm2):
    d, N = 16, 20_000
    x, y = _pair(norm2, 31 + int(norm2 * 4))
    W = oracle.draw_w(4242 + int(norm2 * 100), d * N, d)
    est = _block_estimates(W, x, y, d)
    target = math.exp(x @ y)
    # closed-form iid variance from the Gaussian moment generating function
    var = (math.exp(np.sum((x + y) ** 2)) - 1) * math.exp(2 * x @ y) / d
    z = (est.mean() - target) / math.sqrt(var / N)
    assert abs(z) < 4, z


@pytest.mark.slow
def test_P6_biased_if_norm_term_dropped():
    # sanity of the test's power: without the -|x|^2/2 term the mean is off by
    # exp((|x|^2+|y|^2)/2), far outside 4 sigma
    d, N = 16, 5000
    x, y = _pair(1.0, 7)
    W = oracle.draw_w(555, d * N, d)
    est = _block_estimates(W, x, y, d) * math.exp(0.5 * (x @ x + y @ y))
    var = (math.exp(np.sum((x + y) ** 2)) - 1) * math.exp(2 * x @ y) / d
    z = (est.mean() - math.exp(x @ y)) / math.sqrt(var / N)
    assert abs(z) > 10


@pytest.mark.slow
def test_P7_orthogonal_features_have_lower_variance():
    d, N = 16, 20_000
    x, y = _pair(2.0, 17)
    est_orf = _block_estimates(oracle.draw_w(8080, d * N, d), x, y, d)
    est_iid = _block_estimates(oracle.draw_w_iid(8081, d * N, d), x, y, d)
    ratio = est_orf.var() / est_iid.var()
    assert ratio < 0.9, ratio


# ---------------------------------------------------------------------------
# P8-P11: the FA-part equation (FAVOR+ method page).
# ---------------------------------------------------------------------------
def _inputs(B, H, L, d, m, seed, scale=None):
    rng = _rng(seed)
    scale = d ** -0.25 if scale is None else scale
    Q = rng.standard_normal((B, H, L, d)) * scale
    K = rng.standard_normal((B, H, L, d)) * scale
    V = rng.standard_normal((B, H, L, d))
    W = oracle.draw_w(seed + 1, m, d)
    return Q, K, V, W


def test_P8_ones_in_ones_out():
    Q, K, V, W = _inputs(2, 2, 64, 16, 32, 1)
    ones = np.ones_like(V)
    np.testing.assert_allclose(oracle.bidir(Q, K, ones, W), 1.0, atol=1e-14)
    np.testing.assert_allclose(oracle.causal(Q, K, ones, W), 1.0, atol=1e-14)


def test_P9_rebracketing_equals_quadratic_form():
    Q, K, V, W = _inputs(2, 3, 96, 16, 48, 2)
    np.testing.assert_allclose(oracle.bidir(Q, K, V, W), oracle.brute(Q, K, V, W, False),
                               rtol=1e-12, atol=1e-13)


def test_P10_single_feature_closed_form():
    # m = 1: q' cancels, every output row is the k'-weighted mean of V
    rng = _rng(10)
    L, d = 40, 8
    Q = rng.standard_normal((L, d)) * 0.5
    K = rng.standard_normal((L, d)) * 0.5
    V = rng.standard_normal((L, d))
    w = rng.standard_normal(d)
    kp = np.exp(K @ w - 0.5 * np.sum(K * K, axis=1))
    expect = (kp @ V) / kp.sum()
    out = oracle.bidir(Q, K, V, w[None, :])
    np.testing.assert_allclose(out, np.broadcast_to(expect, out.shape), rtol=1e-12)
    # causal with m = 1: row i is the weighted mean over the first i+1 tokens
    outc = oracle.causal(Q, K, V, w[None, :])
    for i in (0, 5, L - 1):
        e = (kp[:i + 1] @ V[:i + 1]) / kp[:i + 1].sum()
        np.testing.assert_allclose(outc[i], e, rtol=1e-12)


def test_P11_permutation_symmetry():
    Q, K, V, W = _inputs(1, 2, 50, 16, 32, 11)
    out = oracle.bidir(Q, K, V, W)
    p = _rng(3).permutation(50)
    # joint permutation of keys and values leaves the output unchanged
    np.testing.assert_allclose(oracle.bidir(Q, K[..., p, :], V[..., p, :], W), out, rtol=1e-12)
    # permuting queries permutes the output rows
    np.testing.assert_allclose(oracle.bidir(Q[..., p, :], K, V, W), out[..., p, :], rtol=1e-12)


def test_bidir_is_a_convex_combination_of_values():
    Q, K, V, W = _inputs(1, 1, 80, 16, 16, 12)
    out = oracle.bidir(Q, K, V, W)
    assert np.all(out <= V.max(axis=-2, keepdims=True) + 1e-12)
    assert np.all(out >= V.min(axis=-2, keepdims=True) - 1e-12)


# ---------------------------------------------------------------------------
# P12-P14: the masked (causal) form (thesis record abstract: masked
# self-attention; diagonal included).
# ---------------------------------------------------------------------------
def test_P12_causal_equals_masked_brute_force_L128():
    Q, K, V, W = _inputs(8, 8, 128, 64, 256, 12)
    np.testing.assert_allclose(oracle.causal(Q, K, V, W), oracle.brute(Q, K, V, W, True),
                               rtol=1e-12, atol=1e-13)


def test_P13_causal_first_and_last_rows():
    Q, K, V, W = _inputs(2, 2, 70, 16, 32, 13)
    outc = oracle.causal(Q, K, V, W)
    np.testing.assert_allclose(outc[..., 0, :], V[..., 0, :], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(outc[..., -1, :], oracle.bidir(Q, K, V, W)[..., -1, :],
                               rtol=1e-12, atol=1e-13)


def test_P14_causal_prefix_property():
    Q, K, V, W = _inputs(1, 2, 60, 16, 32, 14)
    out = oracle.causal(Q, K, V, W)
    i = 23
    rng = _rng(99)
    Q2, K2, V2 = Q.copy(), K.copy(), V.copy()
    Q2[..., i + 1:, :] += rng.standard_normal(Q2[..., i + 1:, :].shape)
    K2[..., i + 1:, :] += rng.standard_normal(K2[..., i + 1:, :].shape)
    V2[..., i + 1:, :] += rng.standard_normal(V2[..., i + 1:, :].shape)
    out2 = oracle.causal(Q2, K2, V2, W)
    np.testing.assert_array_equal(out2[..., :i + 1, :], out[..., :i + 1, :])
    assert np.max(np.abs(out2[..., i + 1:, :] - out[..., i + 1:, :])) > 1e-3


def test_causal_mask_includes_diagonal():
    # two tokens: row 1 mixes v0 and v1 with weights q1'k0', q1'k1'
    Q, K, V, W = _inputs(1, 1, 2, 16, 16, 15)
    qp = oracle.phi(Q[0, 0], W)
    kp = oracle.phi(K[0, 0], W)
    a0, a1 = qp[1] @ kp[0], qp[1] @ kp[1]
    expect = (a0 * V[0, 0, 0] + a1 * V[0, 0, 1]) / (a0 + a1)
    np.testing.assert_allclose(oracle.causal(Q, K, V, W)[0, 0, 1], expect, rtol=1e-13)


# ---------------------------------------------------------------------------
# P15: convergence toward exact softmax attention as m grows (abstract:
# the features estimate softmax attention).  The exact side is pinned to a
# library routine first.
# ---------------------------------------------------------------------------
def test_softmax_oracle_matches_library_softmax():
    rng = _rng(20)
    Q = rng.standard_normal((2, 30, 8))
    K = rng.standard_normal((2, 30, 8))
    V = rng.standard_normal((2, 30, 8))
    A = scipy.special.softmax(Q @ np.swapaxes(K, -1, -2), axis=-1)
    np.testing.assert_allclose(oracle.softmax_attention(Q, K, V), A @ V, rtol=1e-12)
    mask = np.tril(np.ones((30, 30)))
    S = np.where(mask > 0, Q @ np.swapaxes(K, -1, -2), -np.inf)
    Ac = scipy.special.softmax(S, axis=-1)
    np.testing.assert_allclose(oracle.softmax_attention(Q, K, V, True), Ac @ V, rtol=1e-12)


def _mean_frob(scale, ms, seeds=range(8)):
    errs = []
    for m in ms:
        e = []
        for s in seeds:
            rng = _rng(700 + s)
            Q = rng.standard_normal((256, 16)) * 16 ** -0.25 * scale
            K = rng.standard_normal((256, 16)) * 16 ** -0.25 * scale
            V = rng.standard_normal((256, 16))
            W = oracle.draw_w(9000 + 31 * s + m, m, 16)
            ref = oracle.softmax_attention(Q, K, V)
            e.append(np.linalg.norm(oracle.bidir(Q, K, V, W) - ref) / np.linalg.norm(ref))
        errs.append(np.mean(e))
    return np.array(errs)


@pytest.mark.slow
def test_P15_convergence_to_softmax():
    ms = np.array([16, 64, 256, 1024, 4096])
    err = _mean_frob(0.5, ms)
    slope = np.polyfit(np.log(ms), np.log(err), 1)[0]
    assert -0.6 <= slope <= -0.3, (slope, err)
    assert err[-1] < 0.06, err
    assert np.all(np.diff(err) < 0), err


@pytest.mark.slow
def test_P15_convergence_at_full_input_scale():
    err = _mean_frob(1.0, [16, 65536], seeds=range(4))
    assert err[1] < 0.5 * err[0], err


# ---------------------------------------------------------------------------
# P16: shift invariance, the premise of any exponent stabiliser.
# ---------------------------------------------------------------------------
def test_P16_shift_invariance():
    Q, K, V, W = _inputs(1, 2, 40, 16, 32, 16)
    Qp, Kp = oracle.phi(Q, W), oracle.phi(K, W)
    ref_b = oracle.attend_bidir(Qp, Kp, V)
    ref_c = oracle.attend_causal(Qp, Kp, V)
    rows = np.exp(_rng(1).uniform(-20, 20, size=Qp.shape[:-1]))[..., None]
    for scale_k in (math.exp(-30.0), math.exp(25.0)):
        np.testing.assert_allclose(oracle.attend_bidir(Qp * rows, Kp * scale_k, V), ref_b,
                                   rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(oracle.attend_causal(Qp * rows, Kp * scale_k, V), ref_c,
                                   rtol=1e-12, atol=1e-14)
    # a per-feature shift on K alone is NOT output-invariant
    feat = np.exp(_rng(2).uniform(-3, 3, size=Kp.shape[-1]))
    assert np.max(np.abs(oracle.attend_bidir(Qp, Kp * feat, V) - ref_b)) > 1e-3
    # ... unless the queries carry the inverse shift
    np.testing.assert_allclose(oracle.attend_bidir(Qp / feat, Kp * feat, V), ref_b, rtol=1e-12)


def test_row_rel_err_metric():
    ref = np.array([[1.0, -2.0], [0.5, 0.25]])
    got = ref + np.array([[0.02, 0.0], [0.0, 0.01]])
    assert math.isclose(oracle.row_rel_err(got, ref), 0.02, rel_tol=1e-12)


# ---------------------------------------------------------------------------
# The Gaussian kernel (FAVOR+ method page: the mechanism approximates softmax
# and Gaussian kernels).  G1-G5 pin phi_gaussian and gaussian_attention the
# way P4-P15 pin the softmax side.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("m,d", [(16, 16), (256, 64), (37, 8)])
def test_G1_gaussian_phi_x_dot_phi_minus_x(m, d):
    # exp(w.x - |x|^2) exp(-w.x - |x|^2) = exp(-2|x|^2) per feature, for every W
    rng = _rng(7 * m + d)
    W = rng.standard_normal((m, d)) * 1.3
    X = rng.standard_normal((50, d)) * 0.6
    lhs = np.sum(oracle.phi_gaussian(X, W) * oracle.phi_gaussian(-X, W), axis=1)
    np.testing.assert_allclose(lhs, np.exp(-2 * np.sum(X * X, axis=1)), rtol=1e-13, atol=0)


def test_G1_gaussian_phi_of_zero_and_positivity():
    W = _rng(3).standard_normal((64, 8))
    np.testing.assert_allclose(oracle.phi_gaussian(np.zeros((1, 8)), W), 1 / 8.0, rtol=1e-15)
    assert np.all(oracle.phi_gaussian(_rng(4).standard_normal((20, 8)) * 2, W) > 0)


def test_G2_gaussian_attention_matches_library_softmax():
    # exp(-|q-k|^2/2) = exp(-|q|^2/2) exp(q.k - |k|^2/2): the query factor
    # cancels per row, so the exact Gaussian attention is a softmax over
    # q.k - |k|^2/2 (library routine)
    rng = _rng(21)
    Q = rng.standard_normal((2, 30, 8))
    K = rng.standard_normal((2, 30, 8))
    V = rng.standard_normal((2, 30, 8))
    logits = Q @ np.swapaxes(K, -1, -2) - 0.5 * np.sum(K * K, axis=-1)[..., None, :]
    A = scipy.special.softmax(logits, axis=-1)
    np.testing.assert_allclose(oracle.gaussian_attention(Q, K, V), A @ V, rtol=1e-12)
    mask = np.tril(np.ones((30, 30))) > 0
    Ac = scipy.special.softmax(np.where(mask, logits, -np.inf), axis=-1)
    np.testing.assert_allclose(oracle.gaussian_attention(Q, K, V, True), Ac @ V, rtol=1e-12)


def test_G3_equal_key_norms_make_the_kernels_agree():
    # with every key of the same norm the key factors exp(-|k|^2/2) are one
    # common scalar and the query factors cancel per row: the Gaussian and the
    # softmax FAVOR+ outputs coincide (same W); with unequal norms they differ
    Q, K, V, W = _inputs(1, 2, 48, 16, 64, 23)
    Ku = K / np.linalg.norm(K, axis=-1, keepdims=True) * 0.9
    for f in (oracle.bidir, oracle.causal):
        np.testing.assert_allclose(f(Q, Ku, V, W, kernel="gaussian"), f(Q, Ku, V, W),
                                   rtol=1e-11, atol=1e-13)
        assert np.max(np.abs(f(Q, K * 2, V, W, kernel="gaussian") - f(Q, K * 2, V, W))) > 1e-3


def test_G3_gaussian_ones_rebracketing_and_brute_force():
    Q, K, V, W = _inputs(2, 2, 64, 16, 32, 24)
    ones = np.ones_like(V)
    np.testing.assert_allclose(oracle.bidir(Q, K, ones, W, kernel="gaussian"), 1.0, atol=1e-14)
    np.testing.assert_allclose(oracle.causal(Q, K, ones, W, kernel="gaussian"), 1.0, atol=1e-14)
    np.testing.assert_allclose(oracle.bidir(Q, K, V, W, kernel="gaussian"),
                               oracle.brute(Q, K, V, W, False, kernel="gaussian"), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(oracle.causal(Q, K, V, W, kernel="gaussian"),
                               oracle.brute(Q, K, V, W, True, kernel="gaussian"), rtol=1e-12, atol=1e-13)


def _gauss_block_estimates(W, x, y, d):
    nb = W.shape[0] // d
    px = oracle.phi_gaussian(x[None, :], W)[0].reshape(nb, d) * math.sqrt(W.shape[0] / d)
    py = oracle.phi_gaussian(y[None, :], W)[0].reshape(nb, d) * math.sqrt(W.shape[0] / d)
    return np.sum(px * py, axis=1)


@pytest.mark.slow
@pytest.mark.parametrize("norm2", [0.25, 1.0])
def test_G4_unbiased_gaussian_kernel(norm2):
    d, N = 16, 20_000
    x, y = _pair(norm2, 61 + int(norm2 * 4))
    W = oracle.draw_w(5151 + int(norm2 * 100), d * N, d)
    est = _gauss_block_estimates(W, x, y, d)
    target = math.exp(-0.5 * np.sum((x - y) ** 2))
    # the softmax-kernel iid variance times the square of exp(-(|x|^2+|y|^2)/2)
    var = ((math.exp(np.sum((x + y) ** 2)) - 1) * math.exp(2 * x @ y) / d
           * math.exp(-(x @ x + y @ y)))
    z = (est.mean() - target) / math.sqrt(var / N)
    assert abs(z) < 4, z


@pytest.mark.slow
def test_G5_convergence_to_gaussian_attention():
    # the Gaussian FAVOR+ output approaches the exact Gaussian attention as m grows
    errs = []
    for m in (16, 1024):
        e = []
        for s in range(6):
            rng = _rng(900 + s)
            Q = rng.standard_normal((128, 16)) * 16 ** -0.25 * 0.5
            K = rng.standard_normal((128, 16)) * 16 ** -0.25 * 0.5
            V = rng.standard_normal((128, 16))
            W = oracle.draw_w(9500 + 13 * s + m, m, 16)
            ref = oracle.gaussian_attention(Q, K, V)
            e.append(np.linalg.norm(oracle.bidir(Q, K, V, W, kernel="gaussian") - ref)
                     / np.linalg.norm(ref))
        errs.append(np.mean(e))
    assert errs[1] < 0.25 * errs[0], errs


# ---------------------------------------------------------------------------
# Generalized kernelizable attention with f = ReLU (FAVOR+ method page and
# the paper's abstract name generalized kernelizable attention; f unnamed,
# ReLU is the reading taken).  U1-U5 pin phi_relu, arccos_kernel and
# arccos_attention.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("m,d", [(16, 16), (256, 64), (37, 8)])
def test_U1_relu_features_split_the_projection(m, d):
    # max(s,0) - max(-s,0) = s and max(s,0) max(-s,0) = 0, for every W
    rng = _rng(11 * m + d)
    W = rng.standard_normal((m, d))
    X = rng.standard_normal((40, d))
    p, n = oracle.phi_relu(X, W), oracle.phi_relu(-X, W)
    np.testing.assert_allclose(p - n, X @ W.T / math.sqrt(m), rtol=1e-14, atol=1e-15)
    assert np.all(p * n == 0) and np.all(p >= 0)


def test_U2_arccos_kernel_special_cases_and_monte_carlo():
    rng = _rng(33)
    x = rng.standard_normal(8)
    u = rng.standard_normal(8)
    y = u - (u @ x) / (x @ x) * x               # orthogonal to x
    k = lambda a, b: oracle.arccos_kernel(a[None], b[None])[0, 0]
    assert math.isclose(k(x, x), 0.5 * (x @ x), rel_tol=1e-12)          # E[relu(g)^2] = 1/2
    assert math.isclose(k(x, y), np.linalg.norm(x) * np.linalg.norm(y) / (2 * math.pi), rel_tol=1e-9)
    assert abs(k(x, -x)) < 1e-12
    # against a plain Monte Carlo average over iid Gaussian w (numpy's generator)
    z = rng.standard_normal(8)
    Wmc = np.random.default_rng(34).standard_normal((2_000_000, 8))
    prod = np.maximum(Wmc @ x, 0) * np.maximum(Wmc @ z, 0)
    se = prod.std() / math.sqrt(len(prod))
    assert abs(prod.mean() - k(x, z)) < 4 * se


def test_U3_relu_attention_is_scale_free():
    # phi_R is positively homogeneous: scaling Q or K by a positive factor
    # cancels in D^-1 (a plausible exp- or bias-based feature would not)
    Q, K, V, W = _inputs(1, 2, 48, 16, 64, 31)
    for f in (oracle.bidir, oracle.causal):
        ref = f(Q, K, V, W, kernel="relu")
        np.testing.assert_allclose(f(3.7 * Q, 0.2 * K, V, W, kernel="relu"), ref, rtol=1e-12, atol=1e-13)
    ones = np.ones_like(V)
    np.testing.assert_allclose(oracle.bidir(Q, K, ones, W, kernel="relu"), 1.0, atol=1e-14)
    np.testing.assert_allclose(oracle.causal(Q, K, V, W, kernel="relu"),
                               oracle.brute(Q, K, V, W, True, kernel="relu"), rtol=1e-12, atol=1e-13)


@pytest.mark.slow
def test_U4_unbiased_arccos_kernel():
    d, N = 16, 20_000
    rng = _rng(71)
    x, y = rng.standard_normal(d) * 0.7, rng.standard_normal(d) * 0.7
    W = oracle.draw_w(6161, d * N, d)
    px = oracle.phi_relu(x[None, :], W)[0].reshape(N, d) * math.sqrt(N)
    py = oracle.phi_relu(y[None, :], W)[0].reshape(N, d) * math.sqrt(N)
    est = np.sum(px * py, axis=1)                      # one m = d estimator per block
    target = oracle.arccos_kernel(x[None], y[None])[0, 0]
    z = (est.mean() - target) / (est.std() / math.sqrt(N))
    assert abs(z) < 4, z


@pytest.mark.slow
def test_U5_convergence_to_arccos_attention():
    errs = []
    for m in (16, 2048):
        e = []
        for s in range(6):
            rng = _rng(1300 + s)
            Q = rng.standard_normal((128, 16))
            K = rng.standard_normal((128, 16))
            V = rng.standard_normal((128, 16))
            W = oracle.draw_w(9700 + 13 * s + m, m, 16)
            ref = oracle.arccos_attention(Q, K, V)
            e.append(np.linalg.norm(oracle.bidir(Q, K, V, W, kernel="relu") - ref) / np.linalg.norm(ref))
        errs.append(np.mean(e))
    assert errs[1] < 0.25 * errs[0], errs


# ---------------------------------------------------------------------------
# Backward pass (chain rule through the definitions; the pages print none).
# B1-B4 pin phi_vjp, attend_bidir_vjp, attend_causal_vjp and the composed
# bidir_backward / causal_backward.
# ---------------------------------------------------------------------------
_BWD_CASES = [(k, c) for k in ("softmax", "gaussian", "relu") for c in (False, True)]


def _bwd_inputs(kernel, seed, L=20, d=8):
    m = 64 if kernel == "relu" else 16     # (ReLU: no all-zero first causal row)
    Q, K, V, W = _inputs(1, 2, L, d, m, seed, scale=0.6)
    dO = _rng(seed + 7).standard_normal(V.shape)
    return Q, K, V, W, dO


def _fwd_bwd(causal):
    return ((oracle.causal, oracle.causal_backward) if causal
            else (oracle.bidir, oracle.bidir_backward))


@pytest.mark.parametrize("kernel,causal", _BWD_CASES)
def test_B1_gradients_match_central_differences(kernel, causal):
    # directional derivative of <dO, O> along random directions, h = 1e-6
    Q, K, V, W, dO = _bwd_inputs(kernel, 101 + 2 * causal)
    fwd, bwd = _fwd_bwd(causal)
    grads = bwd(Q, K, V, W, dO, kernel)
    rng = _rng(55)
    h = 1e-6
    for idx in range(3):
        for _ in range(2):
            D = rng.standard_normal(Q.shape)
            plus, minus = [Q, K, V], [Q, K, V]
            plus[idx] = plus[idx] + h * D
            minus[idx] = minus[idx] - h * D
            fd = (np.sum(dO * fwd(*plus, W, kernel)) - np.sum(dO * fwd(*minus, W, kernel))) / (2 * h)
            an = np.sum(grads[idx] * D)
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), (idx, fd, an)


@pytest.mark.parametrize("kernel,causal", _BWD_CASES)
def test_B2_gradients_match_torch_autograd_of_the_quadratic_form(kernel, causal):
    # an independent forward in torch fp64 (features and A = Q'K'^T, masked,
    # O = A V / A 1), differentiated by torch's autograd
    torch = pytest.importorskip("torch")
    Q, K, V, W, dO = _bwd_inputs(kernel, 202 + causal, L=24)
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V)]
    Wt = torch.tensor(W, dtype=torch.float64)
    m = W.shape[0]

    def feat(x):
        s = x @ Wt.T
        if kernel == "relu":
            return torch.relu(s) / math.sqrt(m)
        c = 0.5 if kernel == "softmax" else 1.0
        return torch.exp(s - c * (x * x).sum(-1, keepdim=True)) / math.sqrt(m)

    A = feat(t[0]) @ feat(t[1]).transpose(-1, -2)
    if causal:
        A = torch.tril(A)
    O = (A @ t[2]) / A.sum(-1, keepdim=True)
    (O * torch.tensor(dO)).sum().backward()
    grads = _fwd_bwd(causal)[1](Q, K, V, W, dO, kernel)
    for g, x in zip(grads, t):
        np.testing.assert_allclose(g, x.grad.numpy(), rtol=1e-9, atol=1e-11)


@pytest.mark.parametrize("kernel,causal", _BWD_CASES)
def test_B3_gradient_invariants(kernel, causal):
    Q, K, V, W, dO = _bwd_inputs(kernel, 303 + causal)
    dQ, dK, dV = _fwd_bwd(causal)[1](Q, K, V, W, dO, kernel)
    # each output row is a convex combination of value rows: sum_j dv_j = sum_i dO_i
    np.testing.assert_allclose(dV.sum(-2), dO.sum(-2), rtol=1e-12, atol=1e-12)
    if causal:
        # row 0 is v_0 whatever q_0 is
        assert np.abs(dQ[..., 0, :]).max() <= 1e-14 * np.abs(dQ).max()
    # V with identical rows: O is constant, so Q and K get no gradient
    Vc = np.broadcast_to(V[..., :1, :], V.shape).copy()
    dQc, dKc, _ = _fwd_bwd(causal)[1](Q, K, Vc, W, dO, kernel)
    assert np.abs(dQc).max() <= 1e-12 and np.abs(dKc).max() <= 1e-12
    if kernel == "relu":
        # positive homogeneity: rescaling one query, or every key, leaves O
        np.testing.assert_allclose(np.sum(dQ * Q, -1), 0, atol=1e-12)
        np.testing.assert_allclose(np.sum(dK * K, (-1, -2)), 0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_B4_single_feature_has_no_query_gradient(causal):
    # m = 1: q' is a positive scalar per row and cancels in the division, so
    # O does not depend on Q; dK and dV follow from O_i = sum_j k'_j v_j / sum_j k'_j
    Q, K, V, _ = _inputs(1, 1, 12, 4, 16, 404, scale=0.7)
    W = oracle.draw_w(405, 1, 4)
    dO = _rng(406).standard_normal(V.shape)
    dQ, dK, dV = _fwd_bwd(causal)[1](Q, K, V, W, dO)
    assert np.abs(dQ).max() <= 1e-13
    k = np.exp(K[0, 0] @ W[0] - 0.5 * np.sum(K[0, 0] ** 2, -1))      # (1/sqrt(m) = 1)
    L = len(k)
    mask = np.tril(np.ones((L, L))) if causal else np.ones((L, L))
    Z = mask @ k                                                        # per row i
    O = (mask * k) @ V[0, 0] / Z[:, None]
    # dV_j = sum_i mask_ij k_j dO_i / Z_i ; dk'_j = sum_i mask_ij (v_j - O_i).dO_i / Z_i
    dV_ref = k[:, None] * (mask.T @ (dO[0, 0] / Z[:, None]))
    dkp = np.sum(mask.T[:, :, None] * (V[0, 0][:, None, :] - O[None, :, :]) * (dO[0, 0] / Z[:, None])[None],
                 axis=(1, 2))
    dK_ref = (dkp * k)[:, None] * (W[0][None, :] - K[0, 0])
    np.testing.assert_allclose(dV[0, 0], dV_ref, rtol=1e-12)
    np.testing.assert_allclose(dK[0, 0], dK_ref, rtol=1e-10, atol=1e-13)


# ---------------------------------------------------------------------------
# The masked form's running state (S, z) after a prefix: S1-S2 pin
# causal_state.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kernel", ["softmax", "gaussian", "relu"])
def test_S1_state_gives_the_last_causal_row(kernel):
    # the output of the last token is q'^T S / q'^T z with the state over
    # every token up to it (the prefix-sum form, computed independently)
    Q, K, V, W = _inputs(1, 2, 30, 8, 64, 91)
    S, z = oracle.causal_state(K, V, W, kernel)
    qp = {"softmax": oracle.phi, "gaussian": oracle.phi_gaussian, "relu": oracle.phi_relu}[kernel](
        Q[..., -1, :], W)
    last = np.einsum("...m,...md->...d", qp, S) / np.einsum("...m,...m->...", qp, z)[..., None]
    np.testing.assert_allclose(last, oracle.causal(Q, K, V, W, kernel)[..., -1, :], rtol=1e-12)


def test_S2_state_is_additive_and_z_is_the_ones_column():
    Q, K, V, W = _inputs(2, 1, 25, 8, 32, 92)
    S, z = oracle.causal_state(K, V, W)
    S1, z1 = oracle.causal_state(K[..., :11, :], V[..., :11, :], W)
    S2, z2 = oracle.causal_state(K[..., 11:, :], V[..., 11:, :], W)
    np.testing.assert_allclose(S, S1 + S2, rtol=1e-13)
    np.testing.assert_allclose(z, z1 + z2, rtol=1e-13)
    Sones, _ = oracle.causal_state(K, np.ones_like(V), W)
    np.testing.assert_allclose(Sones, np.broadcast_to(z[..., None], Sones.shape), rtol=1e-13)
