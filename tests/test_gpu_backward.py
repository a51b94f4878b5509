"""GPU parity of the backward pass: favor_bwd_attn (through the C ABI) against
the fp64 oracle's bidir_backward / causal_backward.

Metric: per (b, h), max |gpu - oracle| over the head's gradient divided by the
largest |oracle| entry of that head's gradient, maximised over heads (a
per-row bar does not fit gradients: causal dq_0 is exactly 0).  Bars: 1e-4
for fp32 inputs, 2e-2 for bf16 inputs (bf16 output rounding alone is up to
2^-9 of an entry).  The GPU and the oracle get the same input values and the
same fp32 W bytes.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

import fullsize

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def fv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_kernelized_attention_favor_amd as m
    return m


def _np64(t):
    return t.detach().cpu().double().numpy()


def grad_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(got - ref).max(axis=(-1, -2))
    den = np.abs(ref).max(axis=(-1, -2))
    return float(np.max(num / den))


def _relu_gate_check(name, got, ref, X, W, dXp, tol, tau):
    """ReLU gradients with the gate decided where the pages leave it open.

    The gate [w_r . x > 0] is a floating-point decision: where |w_r . x| is
    within the projection's rounding of 0 (tau |x| |w_r|: 1e-5 for the fp32
    projection of the generic kernels, 2e-3 (reading R25: 4x the fp16
    operands' Cauchy-Schwarz bound 2^-11 |x| |w_r|) for the fp16 operands of the
    matrix cores), the GPU and the oracle may decide it differently, and both
    answers are gradients of the same function (one-sided derivatives at the
    kink).  Rows within the bar are accepted; a row outside it passes only if
    flipping some of its ambiguous gates (at most 10) in the oracle's gradient
    dx = sum_r [w_r . x > 0] dX'_r w_r / sqrt(m) brings it within the bar.
    """
    m = W.shape[0]
    S = X @ W.T
    amb = np.abs(S) <= tau * np.linalg.norm(X, axis=-1, keepdims=True) * np.linalg.norm(W, axis=-1)
    scale = np.abs(ref).max(axis=(-1, -2), keepdims=True)
    row_err = np.abs(got - ref).max(-1) / scale[..., 0]
    for idx in zip(*np.nonzero(row_err > tol)):
        rs = np.nonzero(amb[idx])[0]
        assert 0 < len(rs) <= 10, (name, idx, float(row_err[idx]), len(rs))
        best = np.inf
        for flips in itertools.product((0, 1), repeat=len(rs)):
            alt = ref[idx].copy()
            for r, f in zip(rs, flips):
                if f:
                    sign = -1.0 if S[idx + (r,)] > 0 else 1.0
                    alt += sign * dXp[idx + (r,)] * W[r] / math.sqrt(m)
            best = min(best, np.abs(got[idx] - alt).max() / scale[idx[:-1]][0, 0])
        assert best <= tol, (name, idx, best)


def _case(shape, dtype, seed, kernel):
    B, H, L, d, m = shape
    rng = np.random.default_rng(seed)
    s = d ** -0.25
    q, k, v, do = (rng.standard_normal((B, H, L, d), dtype=np.float32) for _ in range(4))
    q *= np.float32(s)
    k *= np.float32(s)
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    W = oracle.draw_w(seed + 3, m, d).astype(np.float32)
    return tuple(torch.from_numpy(x).to(td) for x in (q, k, v, do)) + (W,)


def _gpu(fv, q, k, v, W, do, causal, kernel):
    out = fv.bwd(q.cuda(), k.cuda(), v.cuda(), torch.from_numpy(W).cuda(), do.cuda(),
                 causal=causal, kernel=kernel)
    torch.cuda.synchronize()
    return out


def _oracle(q, k, v, W, do, causal, kernel):
    f = oracle.causal_backward if causal else oracle.bidir_backward
    return f(_np64(q), _np64(k), _np64(v), W.astype(np.float64), _np64(do), kernel)


SHAPES = [
    (1, 1, 1, 16, 16),
    (1, 2, 17, 32, 48),
    (2, 1, 255, 64, 256),
    (1, 3, 600, 64, 128),      # causal: ten 64-token segments, the last one partial
    (1, 1, 1030, 16, 64),      # causal: seventeen segments, the last six tokens
    (1, 1, 300, 128, 1024),
]


@pytest.mark.parametrize("kernel", ["softmax", "gaussian", "relu"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_shapes(fv, shape, causal, dtype, kernel):
    if kernel == "relu" and shape[4] < 64:
        shape = shape[:4] + (64,)          # (no all-zero ReLU feature rows)
    q, k, v, do, W = _case(shape, dtype, sum(shape) + 7 * causal, kernel)
    got = _gpu(fv, q, k, v, W, do, causal, kernel)
    ref = _oracle(q, k, v, W, do, causal, kernel)
    if kernel == "relu":
        W64 = W.astype(np.float64)
        vjp = oracle.attend_causal_vjp if causal else oracle.attend_bidir_vjp
        dQp, dKp, _ = vjp(oracle.phi_relu(_np64(q), W64), oracle.phi_relu(_np64(k), W64),
                          _np64(v), _np64(do))
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        if name in ("dQ", "dK") and shape[2] == 1:
            # one token: O = v_0 whatever q and k are, so dQ = dK = 0 up to
            # rounding (bf16: the features and T rounded as matrix-core
            # operands leave ~2^-9 of the terms, which cancel exactly here;
            # reading R26: 1e-2 ~ 5 x 2^-9 of the head's dV scale)
            bound = 1e-5 if dtype == "f32" else 1e-2
            assert np.abs(_np64(g)).max() <= bound * np.abs(ref[2]).max()
            continue
        if kernel == "relu" and name != "dV":
            X, dXp = (q, dQp) if name == "dQ" else (k, dKp)
            _relu_gate_check(name, _np64(g), r, _np64(X), W64, dXp, TOL[dtype],
                             1e-5 if dtype == "f32" else 2e-3)
            continue
        err = grad_err(_np64(g), r)
        assert err <= TOL[dtype], (name, err)


# Shapes of the matrix-core backward (bf16, d = 64, m up to 256): single
# tokens, ragged 32- and 64-token tiles, every supported m, many query blocks
# per head (bidirectional) and many segments with a partial last one (causal:
# at least 256 tokens per segment).
MFMA_SHAPES = [
    (1, 1, 1, 64, 64),
    (1, 2, 65, 64, 192),
    (3, 1, 130, 64, 64),
    (1, 1, 4097, 64, 256),
    (2, 3, 500, 64, 128),
    (1, 2, 1000, 64, 256),
]


@pytest.mark.parametrize("kernel", ["softmax", "gaussian", "relu"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", MFMA_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_matrix_core_shapes(fv, shape, causal, kernel):
    B, H, L, d, m = shape
    assert fv.plan_describe(B, H, L, d, m, fv.BF16, causal)[0] == 1   # the matrix-core plan
    test_backward_shapes(fv, shape, causal, "bf16", kernel)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_value_gradient_sums_and_causal_first_row(fv, causal):
    # sum_j dv_j = sum_i dO_i (each output row is a convex combination of
    # value rows); causal dq_0 = 0 (row 0 is v_0); at a size the oracle
    # would take long on
    q, k, v, do, W = _case((1, 2, 4096, 64, 256), "f32", 61 + causal, "softmax")
    dq, dk, dv = _gpu(fv, q, k, v, W, do, causal, "softmax")
    s_dv = _np64(dv).sum(-2)
    s_do = _np64(do).sum(-2)
    assert np.abs(s_dv - s_do).max() <= 1e-4 * np.abs(s_do).max()
    if causal:
        assert np.abs(_np64(dq)[..., 0, :]).max() <= 1e-6 * np.abs(_np64(dq)).max()


def test_backward_constant_values_give_no_query_or_key_gradient(fv):
    q, k, v, do, W = _case((1, 2, 700, 64, 256), "f32", 71, "softmax")
    vc = v[..., :1, :].expand_as(v).contiguous()
    for causal in (False, True):
        dq, dk, _ = _gpu(fv, q, k, vc, W, do, causal, "softmax")
        _, _, dv = _gpu(fv, q, k, v, W, do, causal, "softmax")
        scale = np.abs(_np64(dv)).max()
        assert np.abs(_np64(dq)).max() <= 1e-5 * scale
        assert np.abs(_np64(dk)).max() <= 1e-5 * scale


@pytest.mark.parametrize("causal", [False, True])
def test_backward_bitwise_deterministic(fv, causal):
    q, k, v, do, W = _case((2, 2, 777, 64, 128), "bf16", 81, "softmax")
    a = _gpu(fv, q, k, v, W, do, causal, "softmax")
    b = _gpu(fv, q, k, v, W, do, causal, "softmax")
    for x, y in zip(a, b):
        assert torch.equal(x, y)


FULL_BWD = [("text_bidir", False), ("text_causal", True), ("protein_long", False),
            ("protein_long", True), ("wide_many", False)]


@pytest.mark.parametrize("name,causal", FULL_BWD,
                         ids=[f"{n}-{'causal' if c else 'bidir'}" for n, c in FULL_BWD])
def test_backward_full_size_all_heads(fv, name, causal):
    # The whole workload's backward on the GPU (matrix cores for the d = 64
    # shapes, both forms; generic kernels for d = 128); every head against
    # the oracle, the bar asserted on the worst head of each gradient.
    w = workloads.workload(name)
    if causal:
        w = w.with_(causal=True)
    torch.manual_seed(0)
    q, k, v = workloads.device_qkv(w)
    do = torch.randn_like(q, dtype=torch.float32).to(q.dtype)
    W = oracle.draw_w(w.seed_w, w.m, w.d).astype(np.float32)
    got = fv.bwd(q, k, v, torch.from_numpy(W).cuda(), do, causal=causal)
    torch.cuda.synchronize()
    qf, kf, vf, df, *gf = fullsize.head_slices((q, k, v, do) + tuple(got), w.heads)
    chunk = 4 if (causal and w.L <= 8192) else 1

    def job(h0, h1):
        ref = _oracle(qf[h0:h1], kf[h0:h1], vf[h0:h1], W, df[h0:h1], causal, "softmax")
        return [[grad_err(fullsize.host64(g, h0 + i, h0 + i + 1), r[i][None])
                 for g, r in zip(gf, ref)] for i in range(h1 - h0)]

    errs = np.asarray(fullsize.per_head_rows(w.heads, chunk, job))
    for j, gname in enumerate(("dQ", "dK", "dV")):
        worst, e = fullsize.report(f"backward {w.name} causal={causal} {gname}", errs[:, j])
        assert e <= TOL["bf16"], (gname, worst, e)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_workspace_reuse_and_garbage(fv, causal):
    # Whatever the workspace holds before a call must not change the result.
    q, k, v, do, W = _case((2, 2, 700, 64, 256), "bf16", 91 + causal, "softmax")
    qd, kd, vd, dd = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    Wd = torch.from_numpy(W).cuda()
    ref = fv.bwd(qd, kd, vd, Wd, dd, causal=causal)
    need = fv.bwd_workspace_bytes(2, 2, 700, 64, 256, fv.BF16, causal)
    for fill in (0x00, 0xFF, 0x7F):
        ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda")
        for _ in range(2):
            got = fv.bwd(qd, kd, vd, Wd, dd, causal=causal, workspace=ws)
            torch.cuda.synchronize()
            for a, b in zip(got, ref):
                assert torch.equal(a, b), fill


def test_backward_graph_replays_match_eager(fv):
    # The matrix-core backward captured once and replayed on new inputs.
    shape = (1, 4, 1500, 64, 256)
    cases = [[x.cuda() for x in _case(shape, "bf16", 100 + i, "softmax")[:4]] for i in range(3)]
    W = torch.from_numpy(_case(shape, "bf16", 100, "softmax")[4]).cuda()
    qs, ks, vs, ds = (x.clone() for x in cases[0])
    ws = torch.zeros(fv.bwd_workspace_bytes(1, 4, 1500, 64, 256, fv.BF16, False),
                     dtype=torch.uint8, device="cuda")
    outs = tuple(torch.empty_like(qs) for _ in range(3))
    fv.bwd(qs, ks, vs, W, ds, out=outs, workspace=ws)   # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fv.bwd(qs, ks, vs, W, ds, out=outs, workspace=ws)
    for q, k, v, d in cases[1:] + cases[:1]:
        qs.copy_(q); ks.copy_(k); vs.copy_(v); ds.copy_(d)
        g.replay()
        torch.cuda.synchronize()
        eager = fv.bwd(q, k, v, W, d)
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a, b)


def test_causal_backward_with_key_exponents_climbing_through_a_segment(fv):
    # Keys along the first feature's direction with a growing length: that
    # feature's exponent |w_0| t - t^2 / 2 climbs by ~27 (natural units) over
    # the sequence, so a segment's frame sits far above its first keys and
    # the early queries' factors 2^(s + c - L) are large; the gradients must
    # still match the oracle (matrix cores, bf16).
    B, H, L, d, m = 1, 2, 1200, 64, 128
    rng = np.random.default_rng(71)
    W = oracle.draw_w(72, m, d).astype(np.float32)
    mu = W[0] / np.linalg.norm(W[0])
    ramp = np.linspace(0, 5, L, dtype=np.float32)[:, None]
    k = rng.standard_normal((B, H, L, d)).astype(np.float32) * 0.1 + ramp * mu
    q = rng.standard_normal((B, H, L, d)).astype(np.float32) * 0.3
    v = rng.standard_normal((B, H, L, d)).astype(np.float32)
    do = rng.standard_normal((B, H, L, d)).astype(np.float32)
    q, k, v, do = (torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v, do))
    assert fv.plan_describe(B, H, L, d, m, fv.BF16, True)[0] == 1
    got = _gpu(fv, q, k, v, W, do, True, "softmax")
    ref = _oracle(q, k, v, W, do, True, "softmax")
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.isfinite(g).all(), name
        err = grad_err(_np64(g), r)
        assert err <= TOL["bf16"], (name, err)
