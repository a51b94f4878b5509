"""GPU parity of the on-device draw of W (favor_draw_projection_device, through
the C ABI) against the host draw (favor_draw_projection) and the fp64
oracle's draw (oracle.draw_w): the same stream and stream order, fp64
orthonormalisation on both sides, so W agrees to fp32 rounding."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

SHAPES = [(256, 64), (512, 128), (48, 16), (100, 32), (17, 8), (1, 1), (300, 128), (64, 64)]


@pytest.fixture(scope="module")
def fv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_kernelized_attention_favor_amd as m
    return m


@pytest.mark.parametrize("m,d", SHAPES)
def test_device_draw_matches_host_and_oracle(fv, m, d):
    seed = 1234 + 7 * m + d
    Wd = fv.draw_projection_device(seed, m, d)
    torch.cuda.synchronize()
    Wg = Wd.cpu().numpy().astype(np.float64)
    Wh = fv.draw_projection(seed, m, d).astype(np.float64)
    Wo = oracle.draw_w(seed, m, d)
    scale = np.abs(Wo).max()
    assert np.abs(Wg - Wh).max() <= 2e-6 * scale
    assert np.abs(Wg - Wo).max() <= 2e-6 * scale


@pytest.mark.parametrize("m,d", [(256, 64), (300, 128), (100, 32)])
def test_device_draw_blocks_are_orthogonal(fv, m, d):
    W = fv.draw_projection_device(99, m, d).cpu().numpy().astype(np.float64)
    for r0 in range(0, m, d):
        B = W[r0:r0 + d]
        n = np.linalg.norm(B, axis=1)
        C = (B @ B.T) / np.outer(n, n)
        assert np.abs(C - np.eye(len(B))).max() <= 2e-6


def test_device_draw_is_deterministic_and_seed_dependent(fv):
    a = fv.draw_projection_device(5, 256, 64)
    b = fv.draw_projection_device(5, 256, 64)
    c = fv.draw_projection_device(6, 256, 64)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert not torch.equal(a, c)


def test_forward_with_a_device_drawn_projection(fv):
    rng = np.random.default_rng(3)
    q, k, v = (torch.from_numpy(rng.standard_normal((1, 2, 500, 64), dtype=np.float32) * s)
               .to(torch.bfloat16).cuda() for s in (64 ** -0.25, 64 ** -0.25, 1.0))
    Wd = fv.draw_projection_device(77, 256, 64)
    o = fv.fwd_bidir(q, k, v, Wd)
    torch.cuda.synchronize()
    W64 = oracle.draw_w(77, 256, 64)
    ref = oracle.bidir(*(x.cpu().double().numpy() for x in (q, k, v)), W64)
    assert oracle.row_rel_err(o.cpu().double().numpy(), ref) <= 2e-2
