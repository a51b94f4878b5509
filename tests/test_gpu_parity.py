"""GPU parity: libfavor.so (through its C ABI) against the fp64 oracle.

Metric: max over (b, h, row) of |gpu - oracle|_inf / |oracle|_inf per output
row.  Bars: 1e-4 for fp32 inputs and 2e-2 for bf16 inputs (bf16 output
rounding alone is up to 2^-9 of a row's largest element).  The oracle and the
GPU receive the same input values and the same fp32 W bytes; W comes from the
oracle's draw, never from the library.
"""
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


def _w(seed, m, d):
    return oracle.draw_w(seed, m, d).astype(np.float32)


def _np64(t):
    return t.detach().cpu().double().numpy()


def _run(fv, causal, q, k, v, W):
    Wd = torch.from_numpy(W).cuda()
    out = (fv.fwd_causal if causal else fv.fwd_bidir)(q.cuda(), k.cuda(), v.cuda(), Wd)
    torch.cuda.synchronize()
    return out


def _ref(causal, q, k, v, W):
    f = oracle.causal if causal else oracle.bidir
    return f(_np64(q), _np64(k), _np64(v), W.astype(np.float64))


def _case(B, H, L, d, m, dtype, seed, scale=None):
    rng = np.random.default_rng(seed)
    s = d ** -0.25 if scale is None else scale
    q = rng.standard_normal((B, H, L, d), dtype=np.float32) * np.float32(s)
    k = rng.standard_normal((B, H, L, d), dtype=np.float32) * np.float32(s)
    v = rng.standard_normal((B, H, L, d), dtype=np.float32)
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    return tuple(torch.from_numpy(x).to(td) for x in (q, k, v))


# ---------------------------------------------------------------------------
# Tiny fp32 workload: oracle, V = ones, brute force, exact-softmax trend.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_tiny_f32_workload(fv, causal):
    w = workloads.workload("tiny_f32")
    q, k, v = workloads.host_qkv(w)
    W = _w(w.seed_w, w.m, w.d)
    out = _run(fv, causal, q, k, v, W)
    ref = _ref(causal, q, k, v, W)
    err = oracle.row_rel_err(_np64(out), ref)
    assert err <= TOL["f32"], err
    brute = oracle.brute(_np64(q), _np64(k), _np64(v), W.astype(np.float64), causal)
    assert oracle.row_rel_err(_np64(out), brute) <= TOL["f32"]
    ones = torch.ones_like(v)
    o1 = _run(fv, causal, q, k, ones, W)
    assert np.max(np.abs(_np64(o1) - 1.0)) <= 1e-5


def test_tiny_f32_approaches_softmax_like_the_oracle(fv):
    # With many features the GPU's distance to exact softmax attention equals
    # the oracle's (same W), at reduced input scale where the estimator
    # converges quickly.
    w = workloads.workload("tiny_f32")
    q, k, v = workloads.host_qkv(w)
    q, k = q * 0.5, k * 0.5
    exact = oracle.softmax_attention(_np64(q), _np64(k), _np64(v))
    errs = []
    for m in (16, 1024):
        W = _w(77 + m, m, w.d)
        g = _np64(_run(fv, False, q, k, v, W))
        o = _ref(False, q, k, v, W)
        eg = np.linalg.norm(g - exact) / np.linalg.norm(exact)
        eo = np.linalg.norm(o - exact) / np.linalg.norm(exact)
        assert abs(eg - eo) <= 1e-4 * eo + 1e-6
        errs.append(eg)
    assert errs[1] < 0.5 * errs[0]


# ---------------------------------------------------------------------------
# Shape coverage, fp32 and bf16, with ragged tails.
# ---------------------------------------------------------------------------
SHAPES = [
    # (B, H, L, d, m)
    (1, 1, 1, 16, 16),
    (1, 2, 17, 32, 48),
    (2, 1, 255, 64, 256),
    (1, 1, 600, 128, 1024),
    (1, 3, 1000, 64, 128),
    (1, 1, 4097, 16, 64),
    (1, 1, 2049, 64, 64),     # causal: nine segments, the last one token long
    (2, 2, 333, 64, 192),
    (1, 2, 700, 128, 512),    # bidirectional: two key feature blocks, streamed query side
    (1, 1, 500, 64, 768),     # bidirectional: two key feature blocks, streamed query side
    (1, 2, 300, 128, 256),    # bidirectional: wide heads, query operands resident in LDS
    (1, 1, 1, 64, 256),       # matrix-core path with one token (every tile ragged)
    (1, 3, 31, 64, 256),      # one partial 32-token tile per head
    (1, 1, 33, 128, 512),     # streamed query side with a 1-token second tile
    (3, 1, 257, 64, 128),     # odd head count, one token past a tile boundary
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_shapes(fv, shape, causal, dtype):
    B, H, L, d, m = shape
    q, k, v = _case(B, H, L, d, m, dtype, seed=sum(shape) + causal)
    W = _w(31 * d + m, m, d)
    out = _run(fv, causal, q, k, v, W)
    err = oracle.row_rel_err(_np64(out), _ref(causal, q, k, v, W))
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("causal", [False, True])
def test_text_shape_L128_brute_force(fv, causal):
    # The text configuration's heads and features at L = 128, against the
    # O(L^2) masked (or unmasked) feature attention.
    w = workloads.workload("text_causal")
    q, k, v = workloads.host_qkv(w, L=128)
    W = _w(w.seed_w, w.m, w.d)
    out = _run(fv, causal, q, k, v, W)
    brute = oracle.brute(_np64(q), _np64(k), _np64(v), W.astype(np.float64), causal)
    assert oracle.row_rel_err(_np64(out), brute) <= TOL["bf16"]
    if causal:
        # row 0 is v_0 (up to bf16 output rounding)
        np.testing.assert_allclose(_np64(out)[..., 0, :], _np64(v)[..., 0, :], rtol=8e-3, atol=1e-6)


def test_long_single_head_many_splits(fv):
    # One head of 20000 tokens: 79 key-side splits, the combine's batches of
    # eight splits with a ragged last batch.
    B, H, L, d, m = 1, 1, 20000, 64, 256
    q, k, v = _case(B, H, L, d, m, "bf16", seed=5)
    W = _w(7, m, d)
    out = _run(fv, False, q, k, v, W)
    err = oracle.row_rel_err(_np64(out), _ref(False, q, k, v, W))
    assert err <= TOL["bf16"], err


def test_workspace_reuse_and_garbage(fv):
    # Whatever the workspace holds before a call (never-written memory, an
    # earlier call's partial states) must not change the result.
    B, H, L, d, m = 2, 2, 1500, 64, 256
    q, k, v = _case(B, H, L, d, m, "bf16", seed=3)
    W = torch.from_numpy(_w(11, m, d)).cuda()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    need = fv.workspace_bytes(B, H, L, d, m, 1, False)
    ref = fv.fwd_bidir(qd, kd, vd, W)
    for fill in (0x00, 0xFF, 0x01):
        ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda")
        for _ in range(3):   # the later calls see the counters of the earlier ones
            out = fv.fwd_bidir(qd, kd, vd, W, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(out, ref), fill


def test_graph_replays_match_eager(fv):
    # The forward pass captured once in a HIP graph and replayed on new
    # inputs gives the eager results, replay after replay.
    B, H, L, d, m = 1, 4, 3000, 64, 256
    W = torch.from_numpy(_w(13, m, d)).cuda()
    cases = [[x.cuda() for x in _case(B, H, L, d, m, "bf16", seed=40 + i)] for i in range(4)]
    qs, ks, vs = (x.clone() for x in cases[0])
    ws = torch.zeros(fv.workspace_bytes(B, H, L, d, m, 1, False), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(qs)
    fv.fwd_bidir(qs, ks, vs, W, out=out, workspace=ws)   # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fv.fwd_bidir(qs, ks, vs, W, out=out, workspace=ws)
    for q, k, v in cases[1:] + cases[:1]:
        qs.copy_(q); ks.copy_(k); vs.copy_(v)
        g.replay()
        torch.cuda.synchronize()
        eager = fv.fwd_bidir(q, k, v, W)
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


# ---------------------------------------------------------------------------
# Full-size workloads: the whole launch on the GPU, every head on the oracle.
# ---------------------------------------------------------------------------
FULL = [("text_bidir", False), ("text_causal", True), ("protein_long", False),
        ("protein_long", True), ("wide_many", False)]


def _chunk(w, causal):
    # heads per oracle job: the causal oracle's token loop is vectorised over
    # heads, so short sequences go a few heads at a time
    return 4 if (causal and w.L <= 8192) else 1


def _all_heads(label, w, causal, q, k, v, out, W, ref_fn):
    qf, kf, vf, of = fullsize.head_slices((q, k, v, out), w.heads)

    def job(h0, h1):
        ref = ref_fn(causal, qf[h0:h1], kf[h0:h1], vf[h0:h1], W)
        got = fullsize.host64(of, h0, h1)
        return [oracle.row_rel_err(got[i], ref[i]) for i in range(h1 - h0)]

    errs = fullsize.per_head(w.heads, _chunk(w, causal), job)
    worst, e = fullsize.report(label, errs)
    assert e <= TOL["bf16"], (worst, e)


@pytest.mark.parametrize("name,causal", FULL, ids=[f"{n}-{'causal' if c else 'bidir'}" for n, c in FULL])
def test_full_size_all_heads(fv, name, causal):
    w = workloads.workload(name)
    torch.manual_seed(0)
    q, k, v = workloads.device_qkv(w)
    W = _w(w.seed_w, w.m, w.d)
    out = (fv.fwd_causal if causal else fv.fwd_bidir)(q, k, v, torch.from_numpy(W).cuda())
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    _all_heads(f"{name} causal={causal}", w, causal, q, k, v, out, W, _ref)


# The generic causal path's segments are 64 tokens, doubled (up to 256) while
# the per-segment states would pass 512 MB: these fp32 shapes (m = 1024 is
# beyond the matrix-core forms) take the 128- and 256-token segments.  Every
# head against the oracle at the fp32 bar.
@pytest.mark.parametrize("H,seg", [(16, 128), (32, 256)])
def test_generic_causal_long_segments_all_heads(fv, H, seg):
    B, L, d, m = 1, 8192, 64, 1024
    path, nseg, got_seg = fv.plan_describe(B, H, L, d, m, fv.F32, True)
    assert (path, nseg, got_seg) == (0, L // seg, seg)
    q, k, v = _case(B, H, L, d, m, "f32", seed=80 + H)
    W = _w(90 + H, m, d)
    out = fv.fwd_causal(q.cuda(), k.cuda(), v.cuda(), torch.from_numpy(W).cuda())
    torch.cuda.synchronize()
    qf, kf, vf = (x.reshape(B * H, L, d) for x in (q, k, v))
    of = out.cpu().reshape(B * H, L, d).double().numpy()

    def job(h0, h1):
        ref = _ref(True, qf[h0:h1], kf[h0:h1], vf[h0:h1], W)
        return [oracle.row_rel_err(of[h0 + i], ref[i]) for i in range(h1 - h0)]

    errs = fullsize.per_head(B * H, 4, job)
    worst, e = fullsize.report(f"generic causal, {seg}-token segments", errs)
    assert e <= TOL["f32"], (worst, e)


# ---------------------------------------------------------------------------
# Feature map (projection and exponent arithmetic) and robustness.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_feature_map_closed_form_and_oracle(fv, dtype):
    d, m = 64, 256
    q, _, _ = _case(1, 2, 300, d, m, dtype, seed=5)
    W = _w(9, m, d)
    Wd = torch.from_numpy(W).cuda()
    x = q.cuda()
    p = fv.feature_map(x, Wd)
    pm = fv.feature_map((-x.float()).to(x.dtype).contiguous(), Wd)
    torch.cuda.synchronize()
    lhs = (_np64(p) * _np64(pm)).sum(-1)
    xx = _np64(q)
    np.testing.assert_allclose(lhs, np.exp(-np.sum(xx * xx, -1)), rtol=2e-5)
    np.testing.assert_allclose(_np64(p), oracle.phi(xx, W.astype(np.float64)), rtol=2e-5)


@pytest.mark.parametrize("causal", [False, True])
def test_bitwise_deterministic(fv, causal):
    q, k, v = (x.cuda() for x in _case(2, 4, 1500, 64, 256, "bf16", seed=3))
    W = torch.from_numpy(_w(4, 256, 64)).cuda()
    f = fv.fwd_causal if causal else fv.fwd_bidir
    outs = [f(q, k, v, W).clone() for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


@pytest.mark.parametrize("causal", [False, True])
def test_guard_bands_untouched(fv, causal):
    B, H, L, d, m = 1, 2, 777, 64, 256
    q, k, v = (x.cuda() for x in _case(B, H, L, d, m, "bf16", seed=8))
    W = torch.from_numpy(_w(8, m, d)).cuda()
    n = B * H * L * d
    pad = 4096
    obuf = torch.full((n + 2 * pad,), -12345, dtype=torch.int16, device="cuda")
    out = obuf[pad:pad + n].view(torch.bfloat16).view(B, H, L, d)
    need = fv.workspace_bytes(B, H, L, d, m, fv.BF16, causal)
    wbuf = torch.full((need + 2 * 65536,), 0xA5, dtype=torch.uint8, device="cuda")
    ws = wbuf[65536:65536 + need]
    f = fv.fwd_causal if causal else fv.fwd_bidir
    f(q, k, v, W, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(obuf[:pad] == -12345) and torch.all(obuf[pad + n:] == -12345)
    assert torch.all(wbuf[:65536] == 0xA5) and torch.all(wbuf[65536 + need:] == 0xA5)
    ref = _ref(causal, q, k, v, W.cpu().numpy())
    assert oracle.row_rel_err(_np64(out), ref) <= TOL["bf16"]


def test_causal_prefix_property(fv):
    B, H, L, d, m = 1, 2, 900, 64, 256
    q, k, v = _case(B, H, L, d, m, "bf16", seed=12)
    W = _w(12, m, d)
    out = _np64(_run(fv, True, q, k, v, W))
    i = 400
    g = torch.Generator().manual_seed(1)
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    for t in (q2, k2, v2):
        t[..., i + 1:, :] += torch.randn(t[..., i + 1:, :].shape, generator=g).to(t.dtype)
    out2 = _np64(_run(fv, True, q2, k2, v2, W))
    ref = _ref(True, q, k, v, W)
    assert oracle.row_rel_err(out2[..., :i + 1, :], ref[..., :i + 1, :]) <= TOL["bf16"]
    assert np.max(np.abs(out2[..., i + 1:, :] - out[..., i + 1:, :])) > 1e-2


def test_stabiliser_large_offsets(fv):
    # Exponents far outside fp32's exp range without shifts: Q and K carry a
    # large common offset (|x|^2/2 ~ 300); the oracle in fp64 still holds them.
    B, H, L, d, m = 1, 2, 512, 64, 256
    rng = np.random.default_rng(21)
    mu = rng.standard_normal(d) * 3.0
    q = torch.from_numpy((rng.standard_normal((B, H, L, d)) * 0.35 + mu).astype(np.float32))
    k = torch.from_numpy((rng.standard_normal((B, H, L, d)) * 0.35 + mu).astype(np.float32))
    v = torch.from_numpy(rng.standard_normal((B, H, L, d)).astype(np.float32))
    W = _w(21, m, d)
    for causal in (False, True):
        for dt in (torch.float32, torch.bfloat16):
            qq, kk, vv = q.to(dt), k.to(dt), v.to(dt)
            out = _np64(_run(fv, causal, qq, kk, vv, W))
            ref = _ref(causal, qq, kk, vv, W)
            tol = TOL["f32"] if dt == torch.float32 else TOL["bf16"]
            err = oracle.row_rel_err(out, ref)
            print(f"offset case causal={causal} {dt}: {err:.3e}", flush=True)
            assert err <= tol, (causal, dt, err)


def test_causal_segment_states_redone_with_references(fv):
    # Every key at norm 30: each key exponent w.k - |k|^2/2 lies near -450
    # (natural units), so without references every feature of a segment
    # underflows and its ones-column sum is zero.  The segment-state kernel
    # must then redo the segment with per-feature references.  All keys share
    # the norm, so the |k|^2 term cancels in D^-1 and the output is an
    # ordinary attention that the oracle holds in fp64.  L = 1300 at two heads
    # gives six 224-token segments: five segment states, the last pair of
    # segments with one empty token group.
    B, H, L, d, m = 1, 2, 1300, 64, 256
    rng = np.random.default_rng(77)
    u = rng.standard_normal((B, H, L, d))
    k = 30.0 * u / np.linalg.norm(u, axis=-1, keepdims=True)
    q = rng.standard_normal((B, H, L, d)) * d ** -0.25
    v = rng.standard_normal((B, H, L, d))
    qt, kt, vt = (torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16) for x in (q, k, v))
    W = _w(77, m, d)
    out = _np64(_run(fv, True, qt, kt, vt, W))
    err = oracle.row_rel_err(out, _ref(True, qt, kt, vt, W))
    print(f"norm-30 keys causal: {err:.3e}", flush=True)
    assert np.isfinite(out).all() and err <= TOL["bf16"], err


def test_redraw_changes_output_consistently(fv):
    # Redrawing W (a new seed, uploaded between calls on the same buffers)
    # gives the oracle's result for each W.
    q, k, v = _case(1, 2, 256, 64, 256, "bf16", seed=2)
    outs = []
    for seed in (5002, 5003):
        W = _w(seed, 256, 64)
        out = _run(fv, False, q, k, v, W)
        assert oracle.row_rel_err(_np64(out), _ref(False, q, k, v, W)) <= TOL["bf16"]
        outs.append(_np64(out))
    assert np.max(np.abs(outs[0] - outs[1])) > 1e-3


def test_kernel_timing_records_each_launch(fv):
    w = workloads.workload("text_causal").with_(B=1, H=4, L=3000)
    q, k, v = workloads.host_qkv(w)
    Wd = torch.from_numpy(_w(w.seed_w, w.m, w.d)).cuda()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    for causal, names in ((False, {"kpart", "kcombine", "qapply"}),
                          (True, {"ckey", "kprefix", "cscan"})):
        fwd = fv.fwd_causal if causal else fv.fwd_bidir
        fwd(qd, kd, vd, Wd)
        torch.cuda.synchronize()
        fv.timing_start()
        for _ in range(3):
            fwd(qd, kd, vd, Wd)
        rec = fv.timing_stop()
        assert set(rec) == names, rec
        for name, (ms, launches) in rec.items():
            assert launches == 3 and 0.0 < ms < 1e3, (name, ms, launches)
    # Recording is off after stop: later calls add nothing.
    fv.fwd_bidir(qd, kd, vd, Wd)
    torch.cuda.synchronize()
    fv.timing_start()
    assert fv.timing_stop() == {}


@pytest.mark.parametrize("shape", [(1, 2, 1000, 64, 256), (1, 1, 700, 128, 512), (1, 1, 3000, 64, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_late_exponent_spikes_force_rereferencing(fv, shape):
    # A few keys and queries late in the sequence lie exactly along one
    # projection row: their exponent for that feature, |w|^2 / 2 (about 46
    # log2 units at d = 64), exceeds everything in the first tile or chunk by
    # far more than the kernels' headroom, so the mid-stream re-reference
    # paths (accumulator rescale, already-projected tiles shifted) run.
    B, H, L, d, m = shape
    rng = np.random.default_rng(sum(shape))
    s = d ** -0.25
    q = rng.standard_normal((B, H, L, d)) * s
    k = rng.standard_normal((B, H, L, d)) * s
    v = rng.standard_normal((B, H, L, d))
    W = _w(99 + d + m, m, d)
    # the longest rows give the largest exponents (|w|^2 / 2); queries use
    # rows outside the first 64-feature chunk
    big = np.argsort(-(W.astype(np.float64) ** 2).sum(1))
    late = [f for f in big if f >= 64][:3]
    for j, fk, fq in zip((L // 3, L // 2, L - 3), big[:3], late):
        k[:, :, j, :] = W[fk]
        q[:, :, j + 1, :] = W[fq]
    qt, kt, vt = (torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16) for x in (q, k, v))
    for causal in ((False, True) if d == 64 else (False,)):
        out = _np64(_run(fv, causal, qt, kt, vt, W))
        ref = _ref(causal, qt, kt, vt, W)
        err = oracle.row_rel_err(out, ref)
        print(f"spikes {shape} causal={causal}: {err:.3e}", flush=True)
        assert np.isfinite(out).all() and err <= TOL["bf16"], (causal, err)


# ---------------------------------------------------------------------------
# The Gaussian kernel exp(-|x-y|^2/2) (method page: FAVOR+ approximates
# softmax and Gaussian kernels): the same kernels with key features
# exp(w.k - |k|^2), against the oracle's Gaussian features.
# ---------------------------------------------------------------------------
GAUSS_SHAPES = [
    (1, 2, 17, 32, 48),       # generic path
    (2, 1, 255, 64, 256),     # matrix-core path
    (1, 3, 1000, 64, 128),
    (1, 1, 2049, 64, 64),     # causal: nine segments, the last one token long
    (1, 2, 700, 128, 512),    # streamed query side
    (1, 1, 1, 64, 256),
]


def _gauss_ref(causal, q, k, v, W):
    f = oracle.causal if causal else oracle.bidir
    return f(_np64(q), _np64(k), _np64(v), W.astype(np.float64), kernel="gaussian")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", GAUSS_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gaussian_shapes(fv, shape, causal, dtype):
    B, H, L, d, m = shape
    q, k, v = _case(B, H, L, d, m, dtype, seed=sum(shape) + 77 + causal)
    W = _w(41 * d + m, m, d)
    f = fv.fwd_causal if causal else fv.fwd_bidir
    out = f(q.cuda(), k.cuda(), v.cuda(), torch.from_numpy(W).cuda(), kernel="gaussian")
    torch.cuda.synchronize()
    err = oracle.row_rel_err(_np64(out), _gauss_ref(causal, q, k, v, W))
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gaussian_feature_map_closed_form_and_oracle(fv, dtype):
    d, m = 64, 256
    q, _, _ = _case(1, 2, 300, d, m, dtype, seed=15)
    W = _w(19, m, d)
    Wd = torch.from_numpy(W).cuda()
    x = q.cuda()
    p = fv.feature_map(x, Wd, kernel="gaussian")
    pm = fv.feature_map((-x.float()).to(x.dtype).contiguous(), Wd, kernel="gaussian")
    torch.cuda.synchronize()
    xx = _np64(q)
    np.testing.assert_allclose((_np64(p) * _np64(pm)).sum(-1), np.exp(-2 * np.sum(xx * xx, -1)),
                               rtol=2e-5)
    np.testing.assert_allclose(_np64(p), oracle.phi_gaussian(xx, W.astype(np.float64)), rtol=2e-5)


@pytest.mark.parametrize("causal", [False, True])
def test_gaussian_ones_in_ones_out(fv, causal):
    q, k, _ = _case(1, 4, 1500, 64, 256, "bf16", seed=17)
    ones = torch.ones_like(q)
    f = fv.fwd_causal if causal else fv.fwd_bidir
    out = f(q.cuda(), k.cuda(), ones.cuda(), torch.from_numpy(_w(17, 256, 64)).cuda(),
            kernel="gaussian")
    torch.cuda.synchronize()
    assert torch.all(out.float() == 1.0)


@pytest.mark.parametrize("causal", [False, True])
def test_gaussian_text_shape_all_heads(fv, causal):
    w = workloads.workload("text_causal" if causal else "text_bidir")
    torch.manual_seed(0)
    q, k, v = workloads.device_qkv(w)
    W = _w(w.seed_w, w.m, w.d)
    f = fv.fwd_causal if causal else fv.fwd_bidir
    out = f(q, k, v, torch.from_numpy(W).cuda(), kernel="gaussian")
    torch.cuda.synchronize()
    _all_heads(f"gaussian {w.name} causal={causal}", w, causal, q, k, v, out, W, _gauss_ref)


# ---------------------------------------------------------------------------
# Generalized attention with f = ReLU (paper abstract: generalized kernelizable
# attention): features max(W x, 0)/sqrt(m), the same kernels with no norm term
# and no exponent references, against the oracle's ReLU features.
# ---------------------------------------------------------------------------
RELU_SHAPES = [
    (1, 2, 17, 32, 48),       # generic path
    (2, 1, 255, 64, 256),     # matrix-core path, two token groups per work-group
    (1, 3, 1000, 64, 128),
    (1, 2, 900, 64, 512),     # one token group, 8 waves
    (1, 1, 2049, 64, 64),     # causal: nine segments, the last one token long
    (1, 2, 700, 128, 512),    # streamed query side
    (1, 1, 1, 64, 256),
]


def _relu_ref(causal, q, k, v, W):
    f = oracle.causal if causal else oracle.bidir
    return f(_np64(q), _np64(k), _np64(v), W.astype(np.float64), kernel="relu")


def _relu_run(fv, causal, q, k, v, W):
    f = fv.fwd_causal if causal else fv.fwd_bidir
    out = f(q.cuda(), k.cuda(), v.cuda(), torch.from_numpy(W).cuda(), kernel="relu")
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", RELU_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_relu_shapes(fv, shape, causal, dtype):
    B, H, L, d, m = shape
    q, k, v = _case(B, H, L, d, m, dtype, seed=sum(shape) + 91 + causal)
    W = _w(43 * d + m, m, d)
    out = _relu_run(fv, causal, q, k, v, W)
    err = oracle.row_rel_err(_np64(out), _relu_ref(causal, q, k, v, W))
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_relu_feature_map_split_identity_and_oracle(fv, dtype):
    # max(s, 0) - max(-s, 0) = s: phi(x) - phi(-x) = W x / sqrt(m) for every W
    d, m = 64, 256
    q, _, _ = _case(1, 2, 300, d, m, dtype, seed=16)
    W = _w(23, m, d)
    Wd = torch.from_numpy(W).cuda()
    x = q.cuda()
    p = fv.feature_map(x, Wd, kernel="relu")
    pm = fv.feature_map((-x.float()).to(x.dtype).contiguous(), Wd, kernel="relu")
    torch.cuda.synchronize()
    xx = _np64(q)
    W64 = W.astype(np.float64)
    lin = xx @ W64.T / math.sqrt(m)
    scale = np.abs(lin).max()
    assert np.abs(_np64(p) - _np64(pm) - lin).max() <= 1e-5 * scale
    assert np.all(_np64(p) >= 0) and np.all(_np64(p) * _np64(pm) == 0)
    assert np.abs(_np64(p) - oracle.phi_relu(xx, W64)).max() <= 1e-5 * scale


@pytest.mark.parametrize("causal", [False, True])
def test_relu_scale_free(fv, causal):
    # phi_R is positively homogeneous, so O(a q, b k) = O(q, k) for a, b > 0.
    # fp32 (generic path): powers of two scale every step exactly -> bitwise.
    q, k, v = _case(1, 2, 300, 64, 128, "f32", seed=24)
    W = _w(24, 128, 64)
    o1 = _relu_run(fv, causal, q, k, v, W)
    o2 = _relu_run(fv, causal, q * 4, k * 0.5, v, W)
    assert torch.equal(o1, o2)
    # bf16 (matrix cores): equal to well inside the bar (fp16 subnormals of
    # the projection's operands round differently after scaling)
    q, k, v = _case(2, 2, 1500, 64, 256, "bf16", seed=25)
    W = _w(25, 256, 64)
    o1 = _relu_run(fv, causal, q, k, v, W)
    o2 = _relu_run(fv, causal, q * 4, k * 0.5, v, W)
    err = oracle.row_rel_err(_np64(o2), _np64(o1))
    assert err <= 4e-3, err


@pytest.mark.parametrize("causal", [False, True])
def test_relu_ones_in_ones_out(fv, causal):
    q, k, _ = _case(1, 4, 1500, 64, 256, "bf16", seed=18)
    ones = torch.ones_like(q)
    out = _relu_run(fv, causal, q, k, ones, _w(18, 256, 64))
    assert torch.all(out.float() == 1.0)


@pytest.mark.parametrize("causal", [False, True])
def test_relu_text_shape_all_heads(fv, causal):
    w = workloads.workload("text_causal" if causal else "text_bidir")
    torch.manual_seed(0)
    q, k, v = workloads.device_qkv(w)
    W = _w(w.seed_w, w.m, w.d)
    f = fv.fwd_causal if causal else fv.fwd_bidir
    out = f(q, k, v, torch.from_numpy(W).cuda(), kernel="relu")
    torch.cuda.synchronize()
    _all_heads(f"relu {w.name} causal={causal}", w, causal, q, k, v, out, W, _relu_ref)
