"""GPU parity of the fused bidirectional path (bf16, d = 64, m = 256, at least
64 heads: one persistent kernel after a small preparation launch) against the
fp64 oracle, through the C ABI.

Metric and bar as tests/test_gpu_parity.py: max over rows of
|gpu - oracle|_inf / |oracle|_inf per output row, 2e-2 for bf16 inputs.  Every
head of every case is checked.  Besides shapes (ragged tails, one token,
head counts that give 1 to 4 key splits), the cases force each rare path of
the kernel from its inputs: keys or queries far from every projection row
(the key side's ones column or the query side's denominators underflow
without a reference), a query and keys along the same longest projection row
(the query side's products overflow), and a scaled projection with keys along
a row (the key side's sums overflow).
"""
import numpy as np
import pytest
import torch

import oracle

import fullsize

pytestmark = pytest.mark.gpu

TOL = 2e-2
D, M = 64, 256


@pytest.fixture(scope="module")
def fv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_kernelized_attention_favor_amd as m
    return m


def _w(seed, scale=1.0):
    return (oracle.draw_w(seed, M, D) * scale).astype(np.float32)


def _inputs(B, H, L, seed):
    rng = np.random.default_rng(seed)
    s = np.float32(D ** -0.25)
    q = rng.standard_normal((B, H, L, D), dtype=np.float32) * s
    k = rng.standard_normal((B, H, L, D), dtype=np.float32) * s
    v = rng.standard_normal((B, H, L, D), dtype=np.float32)
    return q, k, v


def _bf16(*xs):
    return tuple(torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
                 for x in xs)


def _effective_w(W):
    """The projection the matrix cores use: fp16(W log2 e) / log2 e (fp64)."""
    log2e = np.float32(1.4426950408889634)
    return (W.astype(np.float32) * log2e).astype(np.float16).astype(np.float64) / float(log2e)


def _check(fv, q, k, v, W, kernel="softmax", label="", W_ref=None):
    B, H, L, d = q.shape
    assert fv.plan_describe(B, H, L, d, W.shape[0], fv.BF16, False)[0] == 2
    out = fv.fwd_bidir(q.cuda(), k.cuda(), v.cuda(), torch.from_numpy(W).cuda(), kernel=kernel)
    torch.cuda.synchronize()
    of = out.cpu().reshape(B * H, L, d)
    qf, kf, vf = (x.reshape(B * H, L, d) for x in (q, k, v))
    W64 = W.astype(np.float64) if W_ref is None else W_ref

    def job(h0, h1):
        ref = oracle.bidir(qf[h0:h1].double().numpy(), kf[h0:h1].double().numpy(),
                           vf[h0:h1].double().numpy(), W64, kernel=kernel)
        got = of[h0:h1].double().numpy()
        return [oracle.row_rel_err(got[i], ref[i]) for i in range(h1 - h0)]

    errs = fullsize.per_head(B * H, 4, job)
    worst, e = fullsize.report(f"fused {label} {tuple(q.shape)} {kernel}", errs)
    assert torch.isfinite(out.float()).all()
    assert e <= TOL, (worst, e)
    return out


SHAPES = [
    (1, 64, 1000),    # four key splits of 256 tokens, ragged last tiles
    (2, 32, 33),      # one 32-token tile and a one-token tile per split
    (1, 64, 1),       # one token per head
    (1, 96, 777),     # three key splits per head
    (1, 256, 300),    # one key split per head
    (1, 64, 5000),    # query blocks of 1280 tokens
    (8, 8, 257),
    (1, 128, 2049),   # two key splits
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fused_shapes(fv, shape):
    B, H, L = shape
    q, k, v = _bf16(*_inputs(B, H, L, sum(shape)))
    _check(fv, q, k, v, _w(11 + L), label="shape")


# (The ReLU features take the three-kernel matrix-core path at these shapes:
# the same calls check it there.)
@pytest.mark.parametrize("kernel", ["gaussian", "relu"])
def test_fused_other_kernels(fv, kernel):
    q, k, v = _bf16(*_inputs(1, 64, 1000, 5))
    _check(fv, q, k, v, _w(6), kernel=kernel, label=kernel)


@pytest.mark.parametrize("kernel", ["softmax", "gaussian", "relu"])
def test_fused_ones_in_ones_out(fv, kernel):
    q, k = _bf16(*_inputs(1, 64, 1500, 7)[:2])
    ones = torch.ones_like(q)
    out = fv.fwd_bidir(q.cuda(), k.cuda(), ones.cuda(), torch.from_numpy(_w(8)).cuda(),
                       kernel=kernel)
    torch.cuda.synchronize()
    assert torch.all(out.float() == 1.0)


def test_fused_bitwise_deterministic_and_workspace_independent(fv):
    # Work items go to whichever work-group takes them first, splits are
    # combined in split order: every call gives the same bits, whatever the
    # workspace held before.
    q, k, v = (x.cuda() for x in _bf16(*_inputs(8, 8, 4096, 9)))
    W = torch.from_numpy(_w(10)).cuda()
    ref = fv.fwd_bidir(q, k, v, W)
    need = fv.workspace_bytes(8, 8, 4096, D, M, fv.BF16, False)
    for fill in (0x00, 0xFF, 0x7F, 0x01):
        ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda")
        for _ in range(3):
            out = fv.fwd_bidir(q, k, v, W, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(out, ref), fill
    for _ in range(20):
        out = fv.fwd_bidir(q, k, v, W)
        assert torch.equal(out, ref)
    torch.cuda.synchronize()


def test_fused_graph_replays_match_eager(fv):
    # The two launches captured once and replayed on new inputs (the control
    # block is cleared by a fill kernel inside the graph).
    B, H, L = 1, 64, 1500
    cases = [tuple(x.cuda() for x in _bf16(*_inputs(B, H, L, 20 + i))) for i in range(3)]
    W = torch.from_numpy(_w(21)).cuda()
    qs, ks, vs = (x.clone() for x in cases[0])
    ws = torch.zeros(fv.workspace_bytes(B, H, L, D, M, fv.BF16, False), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(qs)
    fv.fwd_bidir(qs, ks, vs, W, out=out, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fv.fwd_bidir(qs, ks, vs, W, out=out, workspace=ws)
    for q, k, v in cases[1:] + cases[:1] + cases[1:]:
        qs.copy_(q); ks.copy_(k); vs.copy_(v)
        g.replay()
        torch.cuda.synchronize()
        eager = fv.fwd_bidir(q, k, v, W)
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


def _unit(rng, n):
    x = rng.standard_normal((n, D))
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def test_fused_far_keys_take_the_slow_key_loop(fv):
    # Heads 3 and 40: every key has |k| = 25, so every key feature
    # exp(w.k - |k|^2/2) is below 2^-140 and the fast loop's ones column
    # underflows; those heads' splits are redone with references, and their
    # query tiles then take the slow form (the state carries references).
    # The other heads stay on the fast path.
    q, k, v = _inputs(1, 64, 700, 31)
    rng = np.random.default_rng(32)
    for h in (3, 40):
        k[0, h] = (_unit(rng, 700) * 25.0).astype(np.float32)
    _check(fv, *_bf16(q, k, v), _w(33), label="far keys")


def test_fused_far_queries_take_the_slow_query_tile(fv):
    # Queries with |q| = 25 (some heads, some rows): their features
    # exp(w.q - |q|^2/2) underflow on the fast path, so the tile's
    # denominators fall below 2^-100 and the tile is redone with its exact
    # row maximum as the reference.
    q, k, v = _inputs(1, 64, 900, 41)
    rng = np.random.default_rng(42)
    for h in (0, 17, 63):
        rows = rng.choice(900, size=40, replace=False)
        q[0, h, rows] = (_unit(rng, 40) * 25.0).astype(np.float32)
    _check(fv, *_bf16(q, k, v), _w(43), label="far queries")


def test_fused_aligned_query_and_keys_overflow_to_the_slow_tile(fv):
    # Keys and a query along the longest projection row: each key feature is
    # about 2^(|w|^2 log2(e) / 2) and so is the query's, so their products
    # overflow fp32 on the fast path; the tile is redone with its exact row
    # maximum.
    q, k, v = _inputs(1, 64, 600, 51)
    W = _w(52)
    r = int(np.argmax((W.astype(np.float64) ** 2).sum(1)))
    for h in (5, 6):
        k[0, h, 100:110] = W[r]
        q[0, h, 300] = W[r]
        q[0, h, 599] = W[r]
    _check(fv, *_bf16(q, k, v), W, label="aligned")


def test_fused_scaled_projection_overflows_to_the_slow_key_loop(fv):
    # A projection three times longer than the draw (|w| about 24) and keys
    # of length 12 along one row: those keys' features are about
    # 2^(log2(e) (24 * 12 - 72)) = 2^311, beyond fp32, so the fast loop's
    # sums are not finite and the split is redone with references.
    q, k, v = _inputs(1, 64, 800, 61)
    W = _w(62, scale=3.0)
    r = 7
    u = W[r] / np.linalg.norm(W[r])
    for h in (1, 30):
        k[0, h, 200:204] = (12.0 * u).astype(np.float32)
    _check(fv, *_bf16(q, k, v), W, label="scaled W")


def test_fused_late_exponent_spikes(fv):
    # The spike case of the three-kernel path, on the fused one: a few keys
    # and queries late in the sequence exactly along long projection rows.
    # Their exponents reach |w|^2 log2(e) / 2 (about 70 log2 units), where the
    # fp16 rounding of W log2(e) moves a feature by up to ~2^-12 |s| ln 2
    # (reading R27), so the kernels' own arithmetic is checked against the
    # oracle at the projection they use, fp16(W log2 e) / log2 e, at the bar;
    # against the drawn W the bar is 3e-2.
    B, H, L = 1, 64, 1000
    q, k, v = _inputs(B, H, L, 71)
    W = _w(72)
    big = np.argsort(-(W.astype(np.float64) ** 2).sum(1))
    late = [f for f in big if f >= 64][:3]
    for j, fk, fq in zip((L // 3, L // 2, L - 3), big[:3], late):
        k[:, :, j, :] = W[fk]
        q[:, :, j + 1, :] = W[fq]
    out = _check(fv, *_bf16(q, k, v), W, label="spikes", W_ref=_effective_w(W))
    qf, kf, vf = (x.reshape(B * H, L, D) for x in _bf16(q, k, v))
    of = out.cpu().reshape(B * H, L, D).double().numpy()
    errs = fullsize.per_head(B * H, 4, lambda h0, h1: [
        oracle.row_rel_err(of[h], oracle.bidir(qf[h].double().numpy(), kf[h].double().numpy(),
                                               vf[h].double().numpy(), W.astype(np.float64)))
        for h in range(h0, h1)])
    assert fullsize.report("fused spikes, drawn W", errs)[1] <= 3e-2
