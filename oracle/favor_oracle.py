"""FAVOR+ oracle: a plain, slow, fp64 CPU implementation of what the GPU path computes.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module;
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library (no kernels,
headers, helpers or constant tables) and imports nothing from it.

Sources, by the pages' own titles:

* "Rethinking Attention with Performers" (paper record and abstract on the
  Code with Papers paper page and the mlsanity paper page): positive
  orthogonal random features, unbiased estimation of softmax attention,
  linear space and time.
* "FAVOR+" method page on Code with Papers, section "FAVOR+": the kernel
  definition ``A(i,j) = K(q_i, k_j)`` with ``K(x,y) = E[phi(x)^T phi(y)]``,
  the feature matrices Q', K' whose rows are ``phi(q_i)``, ``phi(k_i)``, and
  the FA-part equation ``Att<-> = D^-1 (Q' ((K')^T V))`` with
  ``D = diag(Q' ((K')^T 1_L))``.
* Performers summary page (aipaper.jasonlin.tech), "Key contributions" and
  "Limitations": positive orthogonal random features; orthogonality holds
  for at most d rows; features are periodically redrawn.
* "Random Features for Efficient Attention Approximation" (thesis record),
  abstract: the masked (causal) self-attention variant and O(L) cost.

Readings where the pages are silent or garbled (each is listed again in the
design notes):

* The diagonal D is printed with ``(K')1_L``; that product does not type-check
  for r != L, so it is read as ``(K')^T 1_L``.
* The method page announces the remaining steps of the mechanism but lists
  none of them, so the feature map itself is not printed.  It is read as the positive softmax-kernel feature
  ``phi(x) = exp(w_r^T x - |x|^2/2) / sqrt(m)``, r = 1..m, which is positive
  and whose expectation over w ~ N(0, I_d) is exactly ``exp(x^T y)``.
* "m <= d" for orthogonality is read as: rows are exactly orthogonal within
  blocks of at most d rows; independent blocks are stacked to reach m.  Row
  norms are drawn independently from chi(d), so each row is marginally
  N(0, I_d).
* The masked form includes the diagonal: token i attends to tokens j <= i.
* The method page says the mechanism approximates softmax and Gaussian
  kernels but prints the features of neither.  For the Gaussian kernel
  ``exp(-|x-y|^2/2) = exp(-|x|^2/2) exp(-|y|^2/2) exp(x^T y)`` the features
  are read as the softmax-kernel features times ``exp(-|x|^2/2)``:
  ``phi_G(x) = exp(w_r^T x - |x|^2) / sqrt(m)``, positive, with expectation
  exactly ``exp(-|x-y|^2/2)``.
* The pages also name generalized kernelizable attention, features
  ``f(W x) / sqrt(m)`` for some f they do not name.  The one built is
  f = ReLU: ``phi_R(x) = max(W x, 0) / sqrt(m)``, non-negative; its
  expectation over w ~ N(0, I_d) is the first-order arc-cosine kernel
  ``|x| |y| (sin t + (pi - t) cos t) / (2 pi)``, t the angle between x and y.
  A query whose features are all zero (e.g. q = 0) has no defined output.
* The backward pass (gradients of the outputs with respect to Q, K and V for
  an upstream gradient dO) is not printed on the pages; it is the plain chain
  rule through the definitions above, with W held fixed (it is redrawn, not
  trained).  The ReLU derivative at exactly 0 is taken as 0.
* The random stream is a counter-based SplitMix64 (Steele, Lea & Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014) feeding the
  Box-Muller transform; the pages name no generator.

No stabiliser is applied here: fp64 holds every exponent the configured
workloads produce, and every public function asserts a finite result with a
positive denominator.

Parity pins (tests/test_oracle_*.py) tie every function here to properties the
pages or the mathematics fix; see the test docstrings for each pin.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "splitmix64",
    "uniforms",
    "normals",
    "draw_w",
    "draw_w_iid",
    "phi",
    "phi_gaussian",
    "phi_relu",
    "attend_bidir",
    "attend_causal",
    "bidir",
    "causal",
    "brute",
    "causal_state",
    "phi_vjp",
    "attend_bidir_vjp",
    "attend_causal_vjp",
    "bidir_backward",
    "causal_backward",
    "softmax_attention",
    "gaussian_attention",
    "arccos_kernel",
    "arccos_attention",
    "row_rel_err",
]

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


# ---------------------------------------------------------------------------
# Random stream: counter-based SplitMix64 (Steele, Lea & Flood 2014).
# Output i of seed s is mix(s + (i + 1) * gamma); mix is the SplitMix64
# finaliser.  Written from the published definition.
# ---------------------------------------------------------------------------
def splitmix64(seed: int, idx: np.ndarray) -> np.ndarray:
    """SplitMix64 output number ``idx`` (uint64 array) of stream ``seed``."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(int(seed) & 0xFFFFFFFFFFFFFFFF) + (idx + np.uint64(1)) * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniforms(seed: int, start: int, count: int) -> np.ndarray:
    """Uniform draws in (0, 1]: the top 53 bits of each output, plus one, times 2^-53."""
    x = splitmix64(seed, np.arange(start, start + count, dtype=np.uint64))
    return ((x >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)


def normals(seed: int, start: int, count: int) -> np.ndarray:
    """Standard normal draws ``start .. start+count-1`` by Box-Muller.

    Normal number n uses uniforms 2*(n//2) and 2*(n//2)+1 (u1, u2); even n
    takes sqrt(-2 ln u1) cos(2 pi u2), odd n the matching sine.
    """
    if count <= 0:
        return np.zeros(0)
    p0 = start // 2
    p1 = (start + count - 1) // 2 + 1
    u = uniforms(seed, 2 * p0, 2 * (p1 - p0)).reshape(-1, 2)
    r = np.sqrt(-2.0 * np.log(u[:, 0]))
    t = 2.0 * math.pi * u[:, 1]
    z = np.empty(2 * (p1 - p0))
    z[0::2] = r * np.cos(t)
    z[1::2] = r * np.sin(t)
    off = start - 2 * p0
    return z[off:off + count]


# ---------------------------------------------------------------------------
# Projection W [m, d]: positive orthogonal random features.
# ---------------------------------------------------------------------------
def draw_w(seed: int, m: int, d: int) -> np.ndarray:
    """Orthogonal Gaussian projection, fp64 [m, d].

    Follows the summary page's "positive orthogonal random features" with the
    block reading: for block b = 0, 1, ... (ceil(m/d) blocks)

    1. G (d x d) takes the next d*d normals of the stream, row-major;
    2. G = QR (Householder QR); U = Q diag(sign(diag R)) makes R's diagonal
       positive, so U is the Gram-Schmidt orthonormalisation of G's columns
       and is Haar-distributed;
    3. the block's rows are the first min(d, m - b d) columns of U;
    4. each row r then takes the next d normals g_r and is scaled by |g_r|,
       a chi(d) draw independent of the direction.
    """
    if m < 1 or d < 1:
        raise ValueError("m and d must be positive")
    W = np.empty((m, d))
    off = 0
    row = 0
    while row < m:
        G = normals(seed, off, d * d).reshape(d, d)
        off += d * d
        Qm, R = np.linalg.qr(G)
        U = Qm * np.sign(np.diag(R))[None, :]
        nb = min(d, m - row)
        g = normals(seed, off, nb * d).reshape(nb, d)   # row i of the block: g[i]
        off += nb * d
        W[row:row + nb] = U[:, :nb].T * np.sqrt(np.sum(g * g, axis=1))[:, None]
        row += nb
    return W


def draw_w_iid(seed: int, m: int, d: int) -> np.ndarray:
    """Unstructured (iid) Gaussian projection, the baseline ORF is compared to."""
    return normals(seed, 0, m * d).reshape(m, d)


# ---------------------------------------------------------------------------
# Feature map and attention.
# ---------------------------------------------------------------------------
def phi(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Positive random features phi(x) = exp(W x - |x|^2 / 2) / sqrt(m).

    X is [..., d], W is [m, d]; the result is [..., m] in fp64.  Rows of the
    result are the rows of Q' or K' in the FA-part equation.
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    m = W.shape[0]
    s = X @ W.T - 0.5 * np.sum(X * X, axis=-1, keepdims=True)
    out = np.exp(s) / math.sqrt(m)
    assert np.all(np.isfinite(out)), "feature exponent out of fp64 range"
    return out


def phi_gaussian(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Positive random features of the Gaussian kernel exp(-|x - y|^2 / 2).

    phi_G(x) = exp(W x - |x|^2) / sqrt(m): the softmax-kernel features times
    exp(-|x|^2 / 2), so that E[phi_G(x)^T phi_G(y)] = exp(-|x - y|^2 / 2).
    Shapes as phi.
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    m = W.shape[0]
    s = X @ W.T - np.sum(X * X, axis=-1, keepdims=True)
    out = np.exp(s) / math.sqrt(m)
    assert np.all(np.isfinite(out)), "feature exponent out of fp64 range"
    return out


def phi_relu(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Generalized (f = ReLU) random features phi_R(x) = max(W x, 0) / sqrt(m).

    Shapes as phi.  E[phi_R(x)^T phi_R(y)] is arccos_kernel(x, y).
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    return np.maximum(X @ W.T, 0.0) / math.sqrt(W.shape[0])


def _features(kernel: str):
    """The feature map of `kernel` ("softmax", "gaussian" or "relu"), looked up at call time."""
    if kernel == "softmax":
        return phi
    if kernel == "gaussian":
        return phi_gaussian
    if kernel == "relu":
        return phi_relu
    raise ValueError(f"unknown kernel {kernel!r}")


def attend_bidir(Qp: np.ndarray, Kp: np.ndarray, V: np.ndarray) -> np.ndarray:
    """FA-part with given features: D^-1 (Q' ((K')^T V)), D = diag(Q' ((K')^T 1_L)).

    Qp, Kp are [..., L, m]; V is [..., L, dv].  The bracketing is the page's:
    (K')^T V first (m x dv), then Q' times it.
    """
    KV = np.swapaxes(Kp, -1, -2) @ V                     # [..., m, dv]
    z = np.sum(Kp, axis=-2)                               # (K')^T 1_L : [..., m]
    num = Qp @ KV                                         # [..., L, dv]
    den = np.einsum("...lm,...m->...l", Qp, z)            # Q' z
    assert np.all(den > 0), "non-positive normaliser"
    out = num / den[..., None]
    assert np.all(np.isfinite(out))
    return out


def attend_causal(Qp: np.ndarray, Kp: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Masked FA-part in prefix-sum form, one token at a time.

    S_i = sum_{j<=i} k'_j v_j^T, z_i = sum_{j<=i} k'_j, out_i = q'_i S_i / q'_i z_i.
    Vectorised over the leading (batch, head) axes only; the loop over tokens
    is sequential, unlike any blocked scan.
    """
    Qp = np.asarray(Qp, dtype=np.float64)
    Kp = np.asarray(Kp, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    lead = Qp.shape[:-2]
    L, m = Qp.shape[-2:]
    dv = V.shape[-1]
    S = np.zeros(lead + (m, dv))
    z = np.zeros(lead + (m,))
    out = np.empty(lead + (L, dv))
    for i in range(L):
        k = Kp[..., i, :]
        S += k[..., :, None] * V[..., i, None, :]
        z += k
        q = Qp[..., i, :]
        num = np.einsum("...m,...md->...d", q, S)
        den = np.einsum("...m,...m->...", q, z)
        assert np.all(den > 0), "non-positive normaliser"
        out[..., i, :] = num / den[..., None]
    assert np.all(np.isfinite(out))
    return out


def bidir(Q, K, V, W, kernel: str = "softmax") -> np.ndarray:
    """Bidirectional FAVOR+ forward: attend_bidir(phi(Q), phi(K), V) in fp64."""
    f = _features(kernel)
    return attend_bidir(f(Q, W), f(K, W), np.asarray(V, dtype=np.float64))


def causal(Q, K, V, W, kernel: str = "softmax") -> np.ndarray:
    """Masked (causal) FAVOR+ forward in prefix-sum form, fp64."""
    f = _features(kernel)
    return attend_causal(f(Q, W), f(K, W), np.asarray(V, dtype=np.float64))


def causal_state(K, V, W, kernel: str = "softmax"):
    """The masked form's running sums after every given token, fp64.

    S = sum_j phi(k_j) v_j^T ([..., m, dv]) and z = sum_j phi(k_j) ([..., m]):
    the state from which the next token's output q'^T S / q'^T z follows.
    """
    Kp = _features(kernel)(K, W)
    V = np.asarray(V, dtype=np.float64)
    return np.swapaxes(Kp, -1, -2) @ V, np.sum(Kp, axis=-2)


def brute(Q, K, V, W, is_causal: bool, kernel: str = "softmax") -> np.ndarray:
    """O(L^2) form: A = Q' K'^T (lower-triangular if masked), out = A V / A 1_L."""
    f = _features(kernel)
    A = f(Q, W) @ np.swapaxes(f(K, W), -1, -2)
    if is_causal:
        L = A.shape[-1]
        A = A * np.tril(np.ones((L, L)))
    den = A.sum(axis=-1)
    assert np.all(den > 0)
    return (A @ np.asarray(V, dtype=np.float64)) / den[..., None]


# ---------------------------------------------------------------------------
# Backward pass: vector-Jacobian products by the chain rule through the
# definitions above (the pages print no backward pass).  For an upstream
# gradient dO of the outputs, each function returns the gradients of
# <dO, O> with respect to its inputs.  W is held fixed.
# ---------------------------------------------------------------------------
def phi_vjp(X, W, G, kernel: str = "softmax") -> np.ndarray:
    """Gradient with respect to X of <G, phi(X)> for the features of `kernel`.

    X is [..., L, d], W [m, d], G [..., L, m].  With Phi = phi(X):
      softmax  d phi_r / dx = phi_r (w_r - x)      -> (G*Phi) W - sum_r(G*Phi) x
      gaussian d phi_r / dx = phi_r (w_r - 2 x)    -> (G*Phi) W - 2 sum_r(G*Phi) x
      relu     d phi_r / dx = [w_r . x > 0] w_r / sqrt(m)
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    if kernel == "relu":
        gate = (X @ W.T > 0).astype(np.float64)
        return ((G * gate) @ W) / math.sqrt(W.shape[0])
    c = {"softmax": 1.0, "gaussian": 2.0}[kernel]
    P = G * _features(kernel)(X, W)
    return P @ W - c * np.sum(P, axis=-1, keepdims=True) * X


def attend_bidir_vjp(Qp, Kp, V, dO):
    """Gradients (dQ', dK', dV) of <dO, attend_bidir(Q', K', V)>.

    Forward in the page's bracketing: S = (K')^T V, z = (K')^T 1_L,
    num = Q' S, den = Q' z, out = num / den.  Backward, step by step:
      dnum = dO / den,  dden = -sum_c dO num / den^2,
      dQ' = dnum S^T + dden z^T,  dS = (Q')^T dnum,  dz = (Q')^T dden,
      dK' = V dS^T + 1_L dz^T,  dV = K' dS.
    """
    Qp, Kp, V, dO = (np.asarray(x, dtype=np.float64) for x in (Qp, Kp, V, dO))
    S = np.swapaxes(Kp, -1, -2) @ V
    z = np.sum(Kp, axis=-2)
    num = Qp @ S
    den = np.einsum("...lm,...m->...l", Qp, z)
    assert np.all(den > 0), "non-positive normaliser"
    dnum = dO / den[..., None]
    dden = -np.sum(dO * num, axis=-1) / den ** 2
    dQp = dnum @ np.swapaxes(S, -1, -2) + dden[..., :, None] * z[..., None, :]
    dS = np.swapaxes(Qp, -1, -2) @ dnum
    dz = np.einsum("...lm,...l->...m", Qp, dden)
    dKp = V @ np.swapaxes(dS, -1, -2) + dz[..., None, :]
    dV = Kp @ dS
    return dQp, dKp, dV


def attend_causal_vjp(Qp, Kp, V, dO):
    """Gradients (dQ', dK', dV) of <dO, attend_causal(Q', K', V)>, token by token.

    A forward sweep rebuilds the prefix states S_i, z_i and gives
    dq'_i = S_i dnum_i + z_i dden_i; a backward sweep over i = L-1 .. 0 keeps
    the suffix sums R_j = sum_{i>=j} q'_i dnum_i^T and r_j = sum_{i>=j} q'_i dden_i,
    which give dk'_j = R_j v_j + r_j and dv_j = R_j^T k'_j.
    """
    Qp, Kp, V, dO = (np.asarray(x, dtype=np.float64) for x in (Qp, Kp, V, dO))
    lead = Qp.shape[:-2]
    L, m = Qp.shape[-2:]
    dv = V.shape[-1]
    dnum = np.empty(lead + (L, dv))
    dden = np.empty(lead + (L,))
    dQp = np.empty(lead + (L, m))
    S = np.zeros(lead + (m, dv))
    z = np.zeros(lead + (m,))
    for i in range(L):
        k = Kp[..., i, :]
        S += k[..., :, None] * V[..., i, None, :]
        z += k
        q = Qp[..., i, :]
        num = np.einsum("...m,...md->...d", q, S)
        den = np.einsum("...m,...m->...", q, z)
        assert np.all(den > 0), "non-positive normaliser"
        dnum[..., i, :] = dO[..., i, :] / den[..., None]
        dden[..., i] = -np.sum(dO[..., i, :] * num, axis=-1) / den ** 2
        dQp[..., i, :] = np.einsum("...md,...d->...m", S, dnum[..., i, :]) + z * dden[..., i, None]
    dKp = np.empty(lead + (L, m))
    dV = np.empty(lead + (L, dv))
    R = np.zeros(lead + (m, dv))
    r = np.zeros(lead + (m,))
    for j in range(L - 1, -1, -1):
        q = Qp[..., j, :]
        R += q[..., :, None] * dnum[..., j, None, :]
        r += q * dden[..., j, None]
        dKp[..., j, :] = np.einsum("...md,...d->...m", R, V[..., j, :]) + r
        dV[..., j, :] = np.einsum("...md,...m->...d", R, Kp[..., j, :])
    return dQp, dKp, dV


def _backward(attend_vjp, Q, K, V, W, dO, kernel):
    f = _features(kernel)
    dQp, dKp, dV = attend_vjp(f(Q, W), f(K, W), V, dO)
    return phi_vjp(Q, W, dQp, kernel), phi_vjp(K, W, dKp, kernel), dV


def bidir_backward(Q, K, V, W, dO, kernel: str = "softmax"):
    """(dQ, dK, dV) of <dO, bidir(Q, K, V, W, kernel)>, fp64."""
    return _backward(attend_bidir_vjp, Q, K, V, W, dO, kernel)


def causal_backward(Q, K, V, W, dO, kernel: str = "softmax"):
    """(dQ, dK, dV) of <dO, causal(Q, K, V, W, kernel)>, fp64."""
    return _backward(attend_causal_vjp, Q, K, V, W, dO, kernel)


def softmax_attention(Q, K, V, is_causal: bool = False) -> np.ndarray:
    """Exact kernel attention with K(x,y) = exp(x^T y), no further scale.

    This is the softmax attention the features estimate; the d^-1/4 factor on
    Q and K (applied by the caller) supplies the usual 1/sqrt(d).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    s = Q @ np.swapaxes(K, -1, -2)
    if is_causal:
        L = s.shape[-1]
        s = np.where(np.tril(np.ones((L, L), dtype=bool)), s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    A = np.exp(s)
    return (A @ V) / A.sum(axis=-1)[..., None]


def gaussian_attention(Q, K, V, is_causal: bool = False) -> np.ndarray:
    """Exact kernel attention with K(x,y) = exp(-|x - y|^2 / 2), no further scale.

    The Gaussian kernel the features phi_G estimate, written from its
    definition: A_ij = exp(-|q_i - k_j|^2 / 2), out = A V / A 1_L (each row
    shifted by its largest exponent, which cancels).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    diff = Q[..., :, None, :] - K[..., None, :, :]
    s = -0.5 * np.sum(diff * diff, axis=-1)
    if is_causal:
        L = s.shape[-1]
        s = np.where(np.tril(np.ones((L, L), dtype=bool)), s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    A = np.exp(s)
    return (A @ V) / A.sum(axis=-1)[..., None]


def arccos_kernel(X, Y) -> np.ndarray:
    """First-order arc-cosine kernel |x| |y| (sin t + (pi - t) cos t) / (2 pi).

    X is [..., n, d], Y is [..., p, d]; the result is [..., n, p].  It is
    E[max(w.x, 0) max(w.y, 0)] for w ~ N(0, I_d) (the half-space integral of
    the Gaussian measure, Cho and Saul 2009), written from its closed form.
    """
    X = np.asarray(X, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    nx = np.linalg.norm(X, axis=-1)[..., :, None]
    ny = np.linalg.norm(Y, axis=-1)[..., None, :]
    cos = np.clip((X @ np.swapaxes(Y, -1, -2)) / np.maximum(nx * ny, 1e-300), -1.0, 1.0)
    t = np.arccos(cos)
    return nx * ny * (np.sin(t) + (math.pi - t) * cos) / (2 * math.pi)


def arccos_attention(Q, K, V, is_causal: bool = False) -> np.ndarray:
    """Exact kernel attention with the arc-cosine kernel: the large-m limit of
    the ReLU features.  A = arccos_kernel(Q, K) (lower-triangular if masked),
    out = A V / A 1_L."""
    A = arccos_kernel(Q, K)
    if is_causal:
        L = A.shape[-1]
        A = A * np.tril(np.ones((L, L)))
    den = A.sum(axis=-1)
    assert np.all(den > 0)
    return (A @ np.asarray(V, dtype=np.float64)) / den[..., None]


def row_rel_err(got, ref) -> float:
    """Parity metric: max over rows of |got - ref|_inf / |ref|_inf (rows = last axis)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-300)
    return float(np.max(num / den))
