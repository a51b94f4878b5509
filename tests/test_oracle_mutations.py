"""The oracle's pins have power: planted mistakes in the oracle fail them.

Each case swaps one oracle function for a plausible wrong version (on the
CPU, inside this process only) and checks that at least one pin from
test_oracle_pins.py then fails.  The real oracle is restored afterwards.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.favor_oracle as fo
import test_oracle_pins as pins

# the real functions, saved before any patching, for mutants built on them
_REAL = {n: getattr(fo, n) for n in ("draw_w", "attend_causal", "softmax_attention",
                                     "gaussian_attention", "arccos_kernel", "phi_vjp",
                                     "attend_bidir_vjp", "attend_causal_vjp")}


def _phi_no_norm(X, W):
    X = np.asarray(X, float)
    return np.exp(X @ np.asarray(W, float).T) / math.sqrt(W.shape[0])


def _phi_plus_norm(X, W):
    X = np.asarray(X, float)
    s = X @ np.asarray(W, float).T + 0.5 * np.sum(X * X, axis=-1, keepdims=True)
    return np.exp(s) / math.sqrt(W.shape[0])


def _phi_no_sqrt_m(X, W):
    X = np.asarray(X, float)
    s = X @ np.asarray(W, float).T - 0.5 * np.sum(X * X, axis=-1, keepdims=True)
    return np.exp(s)


def _draw_unorthogonalised(seed, m, d):
    return fo.normals(seed, 0, m * d).reshape(m, d)


def _draw_fixed_norm(seed, m, d):
    W = _REAL["draw_w"](seed, m, d)
    return W / np.linalg.norm(W, axis=1, keepdims=True) * math.sqrt(d)


def _draw_rows_from_R(seed, m, d):
    # forgets the sign fix: directions are no longer Haar distributed
    W = np.empty((m, d))
    off, row = 0, 0
    while row < m:
        G = fo.normals(seed, off, d * d).reshape(d, d)
        off += d * d
        Qm, _ = np.linalg.qr(G)
        nb = min(d, m - row)
        g = fo.normals(seed, off, nb * d).reshape(nb, d)
        off += nb * d
        W[row:row + nb] = Qm[:nb] * np.sqrt(np.sum(g * g, axis=1))[:, None]
        row += nb
    return W


def _attend_bidir_no_normaliser(Qp, Kp, V):
    return Qp @ (np.swapaxes(Kp, -1, -2) @ V)


def _attend_causal_strict(Qp, Kp, V):
    # excludes the diagonal (j < i), with token 0 attending to itself only
    L = Qp.shape[-2]
    A = Qp @ np.swapaxes(Kp, -1, -2)
    mask = np.tril(np.ones((L, L)), -1)
    mask[0, 0] = 1
    A = A * mask
    return (A @ V) / A.sum(-1)[..., None]


def _attend_causal_off_by_one(Qp, Kp, V):
    # state updated after the output is formed (the diagonal is lost), except row 0
    out = _REAL["attend_causal"](Qp, Kp, V)
    out2 = np.array(out)
    out2[..., 1:, :] = out[..., :-1, :]
    return out2


def _phi_gaussian_half_norm(X, W):
    # the softmax-kernel features under the Gaussian name
    X = np.asarray(X, float)
    s = X @ np.asarray(W, float).T - 0.5 * np.sum(X * X, axis=-1, keepdims=True)
    return np.exp(s) / math.sqrt(W.shape[0])


def _phi_gaussian_double_norm(X, W):
    X = np.asarray(X, float)
    s = X @ np.asarray(W, float).T - 2.0 * np.sum(X * X, axis=-1, keepdims=True)
    return np.exp(s) / math.sqrt(W.shape[0])


def _gaussian_attention_no_half(Q, K, V, is_causal=False):
    # exp(-|q-k|^2) instead of exp(-|q-k|^2/2)
    return _REAL["gaussian_attention"](np.asarray(Q) * math.sqrt(2), np.asarray(K) * math.sqrt(2),
                                       V, is_causal)


def _phi_relu_abs(X, W):
    # |W x| instead of max(W x, 0)
    return np.abs(np.asarray(X, float) @ np.asarray(W, float).T) / math.sqrt(W.shape[0])


def _phi_relu_no_sqrt_m(X, W):
    return np.maximum(np.asarray(X, float) @ np.asarray(W, float).T, 0.0)


def _phi_relu_with_bias(X, W):
    # a small positive floor on every feature (not on the pages)
    return (np.maximum(np.asarray(X, float) @ np.asarray(W, float).T, 0.0) + 1e-3) / math.sqrt(W.shape[0])


def _arccos_t_for_pi_minus_t(X, Y):
    X = np.asarray(X, float)
    Y = np.asarray(Y, float)
    nx = np.linalg.norm(X, axis=-1)[..., :, None]
    ny = np.linalg.norm(Y, axis=-1)[..., None, :]
    cos = np.clip((X @ np.swapaxes(Y, -1, -2)) / (nx * ny), -1.0, 1.0)
    t = np.arccos(cos)
    return nx * ny * (np.sin(t) + t * cos) / (2 * math.pi)


def _softmax_with_scale(Q, K, V, is_causal=False):
    return _REAL["softmax_attention"](np.asarray(Q) / math.sqrt(Q.shape[-1]), K, V, is_causal)




def _run_pins(calls):
    """Return the number of pin calls that fail with an AssertionError."""
    failed = 0
    for f, kw in calls:
        try:
            f(**kw)
        except AssertionError:
            failed += 1
    return failed


PHI_PINS = [
    (pins.test_P4_phi_x_dot_phi_minus_x, dict(m=16, d=16)),
    (pins.test_P5_phi_of_zero, dict(m=16)),
    (pins.test_phi_is_positive_and_matches_single_feature_closed_form, {}),
]
DRAW_PINS = [
    (pins.test_P1_block_orthogonality, dict(m=256, d=64)),
    (pins.test_P2_row_norms_follow_chi_d, dict(d=16)),
    (pins.test_P3_rows_are_marginally_standard_normal, {}),
]
BIDIR_PINS = [
    (pins.test_P8_ones_in_ones_out, {}),
    (pins.test_P9_rebracketing_equals_quadratic_form, {}),
    (pins.test_P10_single_feature_closed_form, {}),
    (pins.test_bidir_is_a_convex_combination_of_values, {}),
]
GAUSS_PINS = [
    (pins.test_G1_gaussian_phi_x_dot_phi_minus_x, dict(m=16, d=16)),
    (pins.test_G1_gaussian_phi_of_zero_and_positivity, {}),
    (pins.test_G3_equal_key_norms_make_the_kernels_agree, {}),
]
RELU_PINS = [
    (pins.test_U1_relu_features_split_the_projection, dict(m=16, d=16)),
    (pins.test_U3_relu_attention_is_scale_free, {}),
]
CAUSAL_PINS = [
    (pins.test_P13_causal_first_and_last_rows, {}),
    (pins.test_causal_mask_includes_diagonal, {}),
    (pins.test_P10_single_feature_closed_form, {}),
]


def _phi_vjp_norm_sign(X, W, G, kernel="softmax"):
    # the norm term's derivative added instead of subtracted
    if kernel == "relu":
        return _REAL["phi_vjp"](X, W, G, kernel)
    X = np.asarray(X, float)
    P = np.asarray(G, float) * fo._features(kernel)(X, W)
    c = {"softmax": 1.0, "gaussian": 2.0}[kernel]
    return P @ np.asarray(W, float) + c * np.sum(P, -1, keepdims=True) * X


def _phi_vjp_relu_no_sqrt_m(X, W, G, kernel="softmax"):
    out = _REAL["phi_vjp"](X, W, G, kernel)
    return out * math.sqrt(W.shape[0]) if kernel == "relu" else out


def _phi_vjp_relu_no_gate(X, W, G, kernel="softmax"):
    if kernel != "relu":
        return _REAL["phi_vjp"](X, W, G, kernel)
    return (np.asarray(G, float) @ np.asarray(W, float)) / math.sqrt(W.shape[0])


def _bidir_vjp_no_dden(Qp, Kp, V, dO):
    # forgets that the normaliser depends on the features too
    S = np.swapaxes(Kp, -1, -2) @ V
    z = np.sum(Kp, axis=-2)
    den = np.einsum("...lm,...m->...l", Qp, z)
    dnum = dO / den[..., None]
    dS = np.swapaxes(Qp, -1, -2) @ dnum
    return dnum @ np.swapaxes(S, -1, -2), V @ np.swapaxes(dS, -1, -2), Kp @ dS


def _bidir_vjp_no_dz(Qp, Kp, V, dO):
    dQp, _, dV = _REAL["attend_bidir_vjp"](Qp, Kp, V, dO)
    S = np.swapaxes(Kp, -1, -2) @ V
    den = np.einsum("...lm,...m->...l", Qp, np.sum(Kp, axis=-2))
    dS = np.swapaxes(Qp, -1, -2) @ (dO / den[..., None])
    return dQp, V @ np.swapaxes(dS, -1, -2), dV


def _causal_vjp_prefix_for_suffix(Qp, Kp, V, dO):
    # the key side sums over earlier queries instead of later ones
    dQp, _, _ = _REAL["attend_causal_vjp"](Qp, Kp, V, dO)
    f = lambda x: np.flip(x, axis=-2)
    _, dKr, dVr = _REAL["attend_causal_vjp"](f(Qp), f(Kp), f(V), f(dO))
    return dQp, f(dKr), f(dVr)


def _causal_vjp_strict_suffix(Qp, Kp, V, dO):
    # the key side skips the diagonal query (i > j instead of i >= j)
    dQp, dKp, dV = _REAL["attend_causal_vjp"](Qp, Kp, V, dO)
    L = Qp.shape[-2]
    Kp2 = np.array(Kp, dtype=float)
    S = np.cumsum(Kp2[..., :, :, None] * np.asarray(V, float)[..., :, None, :], axis=-3)
    z = np.cumsum(Kp2, axis=-2)
    num = np.einsum("...lm,...lmd->...ld", Qp, S)
    den = np.einsum("...lm,...lm->...l", Qp, z)
    dnum = dO / den[..., None]
    dden = -np.sum(dO * num, -1) / den ** 2
    corr_k = Qp * (np.einsum("...ld,...ld->...l", dnum, V) + dden)[..., None]
    corr_v = np.einsum("...lm,...lm->...l", Qp, Kp2)[..., None] * dnum
    return dQp, dKp - corr_k, dV - corr_v


BWD_PINS = [(pins.test_B1_gradients_match_central_differences, dict(kernel=k, causal=c))
            for k, c in pins._BWD_CASES] + [
            (pins.test_B3_gradient_invariants, dict(kernel=k, causal=c)) for k, c in pins._BWD_CASES]


@pytest.mark.parametrize("name,target,mutant", [
    ("feature gradient adds the norm term", "phi_vjp", _phi_vjp_norm_sign),
    ("ReLU feature gradient drops 1/sqrt(m)", "phi_vjp", _phi_vjp_relu_no_sqrt_m),
    ("ReLU feature gradient ignores the gate", "phi_vjp", _phi_vjp_relu_no_gate),
    ("bidirectional gradient drops the normaliser's term", "attend_bidir_vjp", _bidir_vjp_no_dden),
    ("bidirectional key gradient drops dz", "attend_bidir_vjp", _bidir_vjp_no_dz),
    ("causal key side sums over earlier queries", "attend_causal_vjp", _causal_vjp_prefix_for_suffix),
    ("causal key side skips the diagonal", "attend_causal_vjp", _causal_vjp_strict_suffix),
])
def test_planted_backward_mistake_is_caught(monkeypatch, name, target, mutant):
    monkeypatch.setattr(fo, target, mutant)
    assert _run_pins(BWD_PINS) >= 1, f"no pin caught: {name}"


@pytest.mark.parametrize("name,target,mutant,pinset", [
    ("phi drops the norm term", "phi", _phi_no_norm, PHI_PINS),
    ("phi adds the norm term", "phi", _phi_plus_norm, PHI_PINS),
    ("phi drops 1/sqrt(m)", "phi", _phi_no_sqrt_m, PHI_PINS),
    ("draw skips orthogonalisation", "draw_w", _draw_unorthogonalised, DRAW_PINS),
    ("draw fixes norms at sqrt(d)", "draw_w", _draw_fixed_norm, DRAW_PINS),
    ("draw takes rows of Q (no sign fix)", "draw_w", _draw_rows_from_R, DRAW_PINS),
    ("bidir drops the normaliser", "attend_bidir", _attend_bidir_no_normaliser, BIDIR_PINS),
    ("causal excludes the diagonal", "attend_causal", _attend_causal_strict, CAUSAL_PINS),
    ("causal output lags one token", "attend_causal", _attend_causal_off_by_one, CAUSAL_PINS),
    ("Gaussian features keep the softmax norm term", "phi_gaussian", _phi_gaussian_half_norm,
     GAUSS_PINS),
    ("Gaussian features double the norm term", "phi_gaussian", _phi_gaussian_double_norm,
     GAUSS_PINS),
    ("Gaussian attention drops the 1/2", "gaussian_attention", _gaussian_attention_no_half,
     [(pins.test_G2_gaussian_attention_matches_library_softmax, {})]),
    ("ReLU features take |W x|", "phi_relu", _phi_relu_abs, RELU_PINS),
    ("ReLU features drop 1/sqrt(m)", "phi_relu", _phi_relu_no_sqrt_m, RELU_PINS),
    ("ReLU features get a positive floor", "phi_relu", _phi_relu_with_bias, RELU_PINS),
    ("arc-cosine kernel with t for pi - t", "arccos_kernel", _arccos_t_for_pi_minus_t,
     [(pins.test_U2_arccos_kernel_special_cases_and_monte_carlo, {})]),
])
def test_planted_mistake_is_caught(monkeypatch, name, target, mutant, pinset):
    monkeypatch.setattr(fo, target, mutant)
    monkeypatch.setattr(oracle, target, mutant)
    assert _run_pins(pinset) >= 1, f"no pin caught: {name}"


def test_softmax_scale_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(fo, "softmax_attention", _softmax_with_scale)
    monkeypatch.setattr(oracle, "softmax_attention", _softmax_with_scale)
    assert _run_pins([(pins.test_softmax_oracle_matches_library_softmax, {})]) == 1


def test_real_oracle_passes_the_same_pins():
    for pinset in (PHI_PINS, DRAW_PINS, BIDIR_PINS, CAUSAL_PINS, GAUSS_PINS, RELU_PINS, BWD_PINS):
        assert _run_pins(pinset) == 0
