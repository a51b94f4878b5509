"""favor_fwd_attn_noalloc (the forward with the library's static per-GPU
scratch as its workspace) against favor_fwd_attn with a caller workspace,
called through the C ABI: two calls in a row, the second on a smaller input,
each output equal to the existing entry point's (the same kernels, so the same
bits) and within the 2e-2 bf16 bar of the oracle on sampled heads."""
import ctypes

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_kernelized_attention_favor_amd as m
    return m


def _inputs(B, H, L, d, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    q, k, v = (torch.randn((B, H, L, d), generator=g, device="cuda") for _ in range(3))
    s = d ** -0.25
    return (q * s).to(torch.bfloat16), (k * s).to(torch.bfloat16), v.to(torch.bfloat16)


def _noalloc(fv, causal, q, k, v, W, out):
    lib = fv._binding.lib
    B, H, L, d = q.shape
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.favor_fwd_attn_noalloc(B, H, L, d, W.shape[0], fv.BF16, int(causal), fv.SOFTMAX,
                                    q.data_ptr(), k.data_ptr(), v.data_ptr(), W.data_ptr(),
                                    out.data_ptr(), stream)
    assert st == 0, fv.status_string(st)


@pytest.mark.parametrize("causal", [False, True])
def test_noalloc_matches_the_workspace_entry_point(fv, causal):
    d, m = 64, 256
    W = torch.from_numpy(oracle.draw_w(7, m, d).astype(np.float32)).cuda()
    # the text shape's full head count first, then a smaller, ragged input
    for (B, H, L), seed in (((8, 8, 4096), 1), ((1, 3, 1000), 2)):
        q, k, v = _inputs(B, H, L, d, seed)
        out = torch.empty_like(q)
        _noalloc(fv, causal, q, k, v, W, out)
        ref = (fv.fwd_causal if causal else fv.fwd_bidir)(q, k, v, W)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (B, H, L)
        Wn = W.cpu().double().numpy()
        qf, kf, vf, of = (x.reshape(B * H, L, d) for x in (q, k, v, out))
        f = oracle.causal if causal else oracle.bidir
        for h in (0, B * H - 1):
            r = f(*(x[h].cpu().double().numpy() for x in (qf, kf, vf)), Wn)
            err = oracle.row_rel_err(of[h].cpu().double().numpy(), r)
            assert err <= 2e-2, (B, H, L, h, err)


def test_noalloc_rejects_a_shape_beyond_the_scratch(fv):
    # The wide causal shape's workspace is far above the 64 MiB array:
    # refused before anything is enqueued (no pointer is touched).
    lib = fv._binding.lib
    need = fv.workspace_bytes(4, 32, 16384, 128, 512, fv.BF16, True)
    assert need > fv.NOALLOC_SCRATCH_BYTES
    st = lib.favor_fwd_attn_noalloc(4, 32, 16384, 128, 512, fv.BF16, 1, fv.SOFTMAX, 16, 16, 16,
                                    16, 16, None)
    assert st == -8 and "scratch" in fv.status_string(st)
