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
                                     "gaussian_attention", "arccos_kernel")}


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
    for pinset in (PHI_PINS, DRAW_PINS, BIDIR_PINS, CAUSAL_PINS, GAUSS_PINS, RELU_PINS):
        assert _run_pins(pinset) == 0
