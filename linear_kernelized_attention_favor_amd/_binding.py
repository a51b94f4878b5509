"""ctypes binding of libfavor.so (include/favor.h), argument marshalling only.

Every step of the forward pass runs in the HIP library; this module turns
torch tensors into pointers, sizes and the current HIP stream, allocates the
workspace through torch's caching allocator when the caller passes none, and
maps status codes to exceptions.  There is no CPU fallback: if the library is
missing or cannot be loaded, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

__all__ = ["FavorError", "LIB_PATH", "lib", "workspace_bytes", "fwd_bidir", "fwd_causal",
           "fwd_noalloc", "NOALLOC_SCRATCH_BYTES",
           "bwd", "bwd_workspace_bytes", "draw_projection_device", "state_bytes", "state_new", "state_reset", "prefill", "prefill_workspace_bytes",
           "decode",
           "feature_map", "draw_projection", "status_string", "plan_describe", "timing_start", "timing_stop",
           "F32", "BF16", "SOFTMAX", "GAUSSIAN", "RELU"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfavor.so")

F32, BF16 = 0, 1
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}
# attention kernel the features estimate (enum favor_attn_kernel)
SOFTMAX, GAUSSIAN, RELU = 0, 1, 2
_KERNELS = {"softmax": SOFTMAX, "gaussian": GAUSSIAN, "relu": RELU,
            SOFTMAX: SOFTMAX, GAUSSIAN: GAUSSIAN, RELU: RELU}


class FavorError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.favor_status_string(status).decode()
        if status == -6:
            msg += f" (hipError {lib.favor_last_hip_error()})"
        super().__init__(f"{where}: {msg} [status {status}]")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run "
                          "python linear_kernelized_attention_favor_amd/build_lib.py")
    L = ctypes.CDLL(LIB_PATH)
    i32, sz, vp, fp = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p
    L.favor_workspace_bytes.argtypes = [i32] * 7 + [ctypes.POINTER(sz)]
    L.favor_workspace_bytes.restype = ctypes.c_int
    for name in ("favor_fwd_bidir", "favor_fwd_causal"):
        f = getattr(L, name)
        f.argtypes = [i32] * 6 + [vp, vp, vp, fp, vp, vp, sz, vp]
        f.restype = ctypes.c_int
    L.favor_fwd_attn.argtypes = [i32] * 8 + [vp, vp, vp, fp, vp, vp, sz, vp]
    L.favor_fwd_attn.restype = ctypes.c_int
    L.favor_fwd_attn_noalloc.argtypes = [i32] * 8 + [vp, vp, vp, fp, vp, vp]
    L.favor_fwd_attn_noalloc.restype = ctypes.c_int
    L.favor_bwd_workspace_bytes.argtypes = [i32] * 7 + [ctypes.POINTER(sz)]
    L.favor_bwd_workspace_bytes.restype = ctypes.c_int
    L.favor_bwd_attn.argtypes = [i32] * 8 + [vp, vp, vp, fp, vp, vp, vp, vp, vp, sz, vp]
    L.favor_bwd_attn.restype = ctypes.c_int
    L.favor_state_bytes.argtypes = [i32] * 4 + [ctypes.POINTER(sz)]
    L.favor_state_bytes.restype = ctypes.c_int
    L.favor_state_reset.argtypes = [i32] * 4 + [vp, vp]
    L.favor_state_reset.restype = ctypes.c_int
    L.favor_prefill_workspace_bytes.argtypes = [i32] * 6 + [ctypes.POINTER(sz)]
    L.favor_prefill_workspace_bytes.restype = ctypes.c_int
    L.favor_prefill.argtypes = [i32] * 7 + [vp, vp, vp, fp, vp, vp, vp, vp, sz, vp]
    L.favor_prefill.restype = ctypes.c_int
    L.favor_decode.argtypes = [i32] * 6 + [vp, vp, vp, fp, vp, vp, vp]
    L.favor_decode.restype = ctypes.c_int
    L.favor_feature_map.argtypes = [i32] * 6 + [vp, fp, vp, vp]
    L.favor_feature_map.restype = ctypes.c_int
    L.favor_feature_map_attn.argtypes = [i32] * 7 + [vp, fp, vp, vp]
    L.favor_feature_map_attn.restype = ctypes.c_int
    L.favor_draw_projection.argtypes = [ctypes.c_uint64, i32, i32, ctypes.c_void_p]
    L.favor_draw_projection.restype = ctypes.c_int
    L.favor_draw_projection_device.argtypes = [ctypes.c_uint64, i32, i32, vp, vp]
    L.favor_draw_projection_device.restype = ctypes.c_int
    L.favor_status_string.argtypes = [ctypes.c_int]
    L.favor_status_string.restype = ctypes.c_char_p
    L.favor_last_hip_error.argtypes = []
    L.favor_last_hip_error.restype = ctypes.c_int
    L.favor_plan_describe.argtypes = [i32] * 7 + [ctypes.POINTER(i32)] * 3
    L.favor_plan_describe.restype = ctypes.c_int
    L.favor_timing_start.argtypes = []
    L.favor_timing_start.restype = ctypes.c_int
    L.favor_timing_stop.argtypes = [i32, ctypes.POINTER(ctypes.c_char_p),
                                    ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32),
                                    ctypes.POINTER(i32)]
    L.favor_timing_stop.restype = ctypes.c_int
    return L


lib = _load()


def status_string(status: int) -> str:
    return lib.favor_status_string(status).decode()


def _check(status: int, where: str):
    if status != 0:
        raise FavorError(status, where)


def workspace_bytes(B, H, L, d, m, dtype=BF16, causal=False) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.favor_workspace_bytes(B, H, L, d, m, dtype, int(bool(causal)), ctypes.byref(out)),
           "favor_workspace_bytes")
    return out.value


def bwd_workspace_bytes(B, H, L, d, m, dtype=BF16, causal=False) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.favor_bwd_workspace_bytes(B, H, L, d, m, dtype, int(bool(causal)),
                                         ctypes.byref(out)), "favor_bwd_workspace_bytes")
    return out.value


def plan_describe(B, H, L, d, m, dtype=BF16, causal=False):
    """(path, nseg, seg) of the plan a forward call would use (favor_plan_describe)."""
    a, b, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib.favor_plan_describe(B, H, L, d, m, dtype, int(bool(causal)), ctypes.byref(a),
                                   ctypes.byref(b), ctypes.byref(c)), "favor_plan_describe")
    return a.value, b.value, c.value


def _shape_of(q, k, v, W):
    if q.dim() != 4:
        raise ValueError("Q, K, V must be [B, H, L, d]")
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("Q, K, V must share shape, dtype and device")
    for t in (q, k, v, W):
        if not t.is_cuda:
            raise ValueError("tensors must be in GPU memory")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    if W.dtype != torch.float32 or W.dim() != 2 or W.shape[1] != q.shape[3]:
        raise ValueError("W must be fp32 [m, d]")
    if q.dtype not in _DTYPES:
        raise ValueError("inputs must be float32 or bfloat16")
    B, H, L, d = q.shape
    return B, H, L, d, W.shape[0], _DTYPES[q.dtype]


def _stream(q, stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _kernel(kernel):
    try:
        return _KERNELS[kernel]
    except KeyError:
        raise ValueError(f"kernel must be 'softmax', 'gaussian' or 'relu', not {kernel!r}") from None


def _check_out(out, shape, dtype, device, what):
    if (tuple(out.shape) != tuple(shape) or out.dtype != dtype or not out.is_contiguous()
            or not out.is_cuda or out.device != device):
        raise ValueError(f"{what} must be a contiguous {dtype} GPU tensor of shape "
                         f"{list(shape)} on {device}")


def _forward(name, causal, q, k, v, W, out, workspace, stream, kernel="softmax"):
    ak = _kernel(kernel)
    B, H, L, d, m, dt = _shape_of(q, k, v, W)
    need = workspace_bytes(B, H, L, d, m, dt, causal)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, q.shape, q.dtype, q.device, "out")
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), W.data_ptr(), out.data_ptr(),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q, stream))
    if ak == SOFTMAX:
        st = getattr(lib, name)(B, H, L, d, m, dt, *ptrs)
    else:
        name = "favor_fwd_attn"
        st = lib.favor_fwd_attn(B, H, L, d, m, dt, int(causal), ak, *ptrs)
    _check(st, name)
    return out


NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024   # FAVOR_NOALLOC_SCRATCH_BYTES


def fwd_noalloc(q, k, v, W, out, causal=False, kernel="softmax", stream=None):
    """favor_fwd_attn_noalloc: the forward pass into a caller-supplied `out`, with the
    library's static per-GPU scratch as the workspace (nothing is allocated; calls
    that overlap on one GPU race on the scratch)."""
    ak = _kernel(kernel)
    B, H, L, d, m, dt = _shape_of(q, k, v, W)
    _check_out(out, q.shape, q.dtype, q.device, "out")
    st = lib.favor_fwd_attn_noalloc(B, H, L, d, m, dt, int(bool(causal)), ak, q.data_ptr(),
                                    k.data_ptr(), v.data_ptr(), W.data_ptr(), out.data_ptr(),
                                    _stream(q, stream))
    _check(st, "favor_fwd_attn_noalloc")
    return out


def bwd(q, k, v, W, do, causal=False, kernel="softmax", out=None, workspace=None, stream=None):
    """Backward pass (favor_bwd_attn): (dQ, dK, dV), the gradients of <do, O> for the
    forward fwd_causal (causal=True) or fwd_bidir with the same kernel; W is held fixed.
    out, if given, is a tuple of three contiguous tensors like Q."""
    ak = _kernel(kernel)
    B, H, L, d, m, dt = _shape_of(q, k, v, W)
    if do.shape != q.shape or do.dtype != q.dtype or not do.is_contiguous() or not do.is_cuda:
        raise ValueError("do must be a contiguous GPU tensor like Q")
    need = bwd_workspace_bytes(B, H, L, d, m, dt, causal)
    if out is None:
        out = tuple(torch.empty_like(q) for _ in range(3))
    elif len(out) != 3:
        raise ValueError("out must be three contiguous tensors like Q")
    for o in out:
        _check_out(o, q.shape, q.dtype, q.device, "each of out")
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    st = lib.favor_bwd_attn(B, H, L, d, m, dt, int(bool(causal)), ak, q.data_ptr(), k.data_ptr(),
                            v.data_ptr(), W.data_ptr(), do.data_ptr(), out[0].data_ptr(),
                            out[1].data_ptr(), out[2].data_ptr(), workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), _stream(q, stream))
    _check(st, "favor_bwd_attn")
    return out


def state_bytes(B, H, d, m) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.favor_state_bytes(B, H, d, m, ctypes.byref(out)), "favor_state_bytes")
    return out.value


def state_reset(state, stream=None):
    """Empty the causal states in `state` (fp32 [B, H, m, d+4]) on the GPU."""
    if state.dim() != 4 or state.dtype != torch.float32 or not state.is_contiguous():
        raise ValueError("state must be a contiguous fp32 [B, H, m, d+4] tensor")
    B, H, m, d4 = state.shape
    _check(lib.favor_state_reset(B, H, d4 - 4, m, state.data_ptr(), _stream(state, stream)),
           "favor_state_reset")
    return state


def state_new(B, H, d, m, device="cuda"):
    """A new empty causal state for B*H heads: fp32 [B, H, m, d+4] rows [S~ | z~ | c]."""
    st = torch.empty((B, H, m, d + 4), dtype=torch.float32, device=device)
    return state_reset(st)


def _check_state(st, B, H, d, m, what):
    if st is not None and (st.shape != (B, H, m, d + 4) or st.dtype != torch.float32
                           or not st.is_contiguous() or not st.is_cuda):
        raise ValueError(f"{what} must be a contiguous fp32 GPU tensor [B, H, m, d+4]")


def _overlap(a, b) -> bool:
    a0, b0 = a.data_ptr(), b.data_ptr()
    return a0 < b0 + b.numel() * b.element_size() and b0 < a0 + a.numel() * a.element_size()


def prefill_workspace_bytes(B, H, L, d, m, dtype=BF16) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.favor_prefill_workspace_bytes(B, H, L, d, m, dtype, ctypes.byref(n)),
           "favor_prefill_workspace_bytes")
    return n.value


def prefill(q, k, v, W, state_in=None, state_out=None, kernel="softmax", out=None,
            workspace=None, stream=None):
    """Causal forward over new tokens continuing state_in (None: empty) (favor_prefill).

    Returns (O, state_out); state_out is allocated when not given."""
    ak = _kernel(kernel)
    B, H, L, d, m, dt = _shape_of(q, k, v, W)
    _check_state(state_in, B, H, d, m, "state_in")
    if state_out is None:
        state_out = torch.empty((B, H, m, d + 4), dtype=torch.float32, device=q.device)
    _check_state(state_out, B, H, d, m, "state_out")
    if state_in is not None and _overlap(state_in, state_out):
        raise ValueError("state_out must not overlap state_in: the library reads the imported "
                         "state while it writes the exported one (pass a second state buffer "
                         "and swap the two between chunks)")
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, q.shape, q.dtype, q.device, "out")
    if workspace is None:
        need = prefill_workspace_bytes(B, H, L, d, m, dt)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    st = lib.favor_prefill(B, H, L, d, m, dt, ak, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                           W.data_ptr(), out.data_ptr(),
                           None if state_in is None else state_in.data_ptr(),
                           state_out.data_ptr(), workspace.data_ptr(),
                           workspace.numel() * workspace.element_size(), _stream(q, stream))
    _check(st, "favor_prefill")
    return out, state_out


def decode(q, k, v, W, state, kernel="softmax", out=None, stream=None):
    """One decoding step (favor_decode): q, k, v [B, H, d] (one new token per head);
    `state` is updated in place; returns o [B, H, d]."""
    ak = _kernel(kernel)
    if q.dim() != 3:
        raise ValueError("q, k, v must be [B, H, d]")
    B, H, L, d, m, dt = _shape_of(q[:, :, None], k[:, :, None], v[:, :, None], W)
    _check_state(state, B, H, d, m, "state")
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, q.shape, q.dtype, q.device, "out")
    _check(lib.favor_decode(B, H, d, m, dt, ak, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                            W.data_ptr(), out.data_ptr(), state.data_ptr(), _stream(q, stream)),
           "favor_decode")
    return out


def fwd_bidir(q, k, v, W, out=None, workspace=None, stream=None, kernel="softmax"):
    """Bidirectional FAVOR+ forward (enqueued on the current stream): favor_fwd_bidir,
    or favor_fwd_attn for kernel="gaussian" (features of exp(-|x-y|^2/2)) or
    kernel="relu" (features max(W x, 0)/sqrt(m), generalized attention)."""
    return _forward("favor_fwd_bidir", False, q, k, v, W, out, workspace, stream, kernel)


def fwd_causal(q, k, v, W, out=None, workspace=None, stream=None, kernel="softmax"):
    """Causal FAVOR+ forward in prefix-sum form: favor_fwd_causal, or favor_fwd_attn
    for kernel="gaussian" or "relu"."""
    return _forward("favor_fwd_causal", True, q, k, v, W, out, workspace, stream, kernel)


def feature_map(x, W, out=None, stream=None, kernel="softmax"):
    """phi(x) = exp(W x - c |x|^2)/sqrt(m) as fp32 [B, H, L, m], c = 1/2 (softmax,
    favor_feature_map) or 1 (gaussian, favor_feature_map_attn), or
    max(W x, 0)/sqrt(m) (relu, favor_feature_map_attn)."""
    ak = _kernel(kernel)
    B, H, L, d, m, dt = _shape_of(x, x, x, W)
    if out is None:
        out = torch.empty((B, H, L, m), dtype=torch.float32, device=x.device)
    _check_out(out, (B, H, L, m), torch.float32, x.device, "out")
    args = (x.data_ptr(), W.data_ptr(), out.data_ptr(), _stream(x, stream))
    if ak == SOFTMAX:
        st = lib.favor_feature_map(B, H, L, d, m, dt, *args)
        _check(st, "favor_feature_map")
    else:
        st = lib.favor_feature_map_attn(B, H, L, d, m, dt, ak, *args)
        _check(st, "favor_feature_map_attn")
    return out


def draw_projection(seed: int, m: int, d: int) -> np.ndarray:
    """Host draw of the orthogonal projection W [m, d] (fp32), favor_draw_projection."""
    W = np.empty((m, d), dtype=np.float32)
    _check(lib.favor_draw_projection(ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), m, d,
                                     W.ctypes.data_as(ctypes.c_void_p)), "favor_draw_projection")
    return W


def draw_projection_device(seed: int, m: int, d: int, out=None, device="cuda", stream=None):
    """On-device draw of W [m, d] (fp32 GPU tensor), favor_draw_projection_device: the
    host draw's distribution and random stream, enqueued on the current stream."""
    if out is None:
        out = torch.empty((m, d), dtype=torch.float32, device=device)
    elif out.shape != (m, d) or out.dtype != torch.float32 or not out.is_contiguous() \
            or not out.is_cuda:
        raise ValueError("out must be a contiguous fp32 GPU tensor [m, d]")
    _check(lib.favor_draw_projection_device(ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), m, d,
                                            out.data_ptr(), _stream(out, stream)),
           "favor_draw_projection_device")
    return out


def timing_start() -> None:
    """Start recording per-kernel HIP events for this thread's forward calls."""
    _check(lib.favor_timing_start(), "favor_timing_start")


def timing_stop(max_kernels: int = 16) -> dict:
    """Stop recording; {kernel name: (total ms, launches)} in order of first launch."""
    names = (ctypes.c_char_p * max_kernels)()
    ms = (ctypes.c_float * max_kernels)()
    cnt = (ctypes.c_int32 * max_kernels)()
    n = ctypes.c_int32(0)
    _check(lib.favor_timing_stop(max_kernels, names, ms, cnt, ctypes.byref(n)), "favor_timing_stop")
    return {names[k].decode(): (float(ms[k]), int(cnt[k])) for k in range(min(n.value, max_kernels))}
