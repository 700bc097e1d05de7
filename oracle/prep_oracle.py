"""fp64 CPU oracle for the producer of the attention's inputs.

TEST INFRASTRUCTURE. Only the tests, the package's smoke() check and the
benchmark's cpu_baseline leg may import or call this module. The product path
never does, and this module imports nothing from the product.

Source: the page "HeyGen 与 Google Cloud：将 Avatar IV 部署到 TPU"
(news.xcc.im/article/5328), section "Layout Is the ABI" ¶2: the attention's
inputs come out of a chain of small operations (normalization, rotary
embeddings, projections, head packing), which the authors fuse into one kernel
that writes its output in exactly the layout its consumer wants. Here the
consumer is the frame-aligned attention, whose layout is [B][H][N][d] with
tokens frame-major ("Hiding the Collective" ¶2: the mask is defined over that
token order), and which also wants per-row query norms and per-head key sums
for its Cauchy-Schwarz bounds ("Unchaining the Softmax" ¶2).

The page names the operations but not their forms. Readings (each listed in
the design notes):
  * normalization: RMSNorm of each token over its C = H*d channels with a
    learned weight gamma, eps = 1e-6;
  * projections: one linear map without bias, W of shape [3C, C] in the
    (out, in) convention, rows [0, C) for queries, [C, 2C) keys, [2C, 3C)
    values; y = W x_hat;
  * head packing: head h takes channels [h*d, (h+1)*d) of each projection;
  * rotary embeddings: 3-D over the token's (frame t, row y, column x) on a
    latent grid of Hg x Wg patches per frame (T = Hg*Wg, token n lies at
    t = n // T, y = (n % T) // Wg, x = n % Wg); the head width splits into
    bands of d/4 (t), 3d/8 (y) and 3d/8 (x) channels; inside a band of n_b
    channels with coordinate p, channel pair (2i, 2i+1) turns by the angle
    p * BASE**(-2i / n_b), BASE = 10000; applied to queries and keys only.

Precision: float64 numpy throughout.

Pins (tests/test_prep_oracle.py): torch's rms_norm and linear in float64,
explicit loops on a tiny case, the rotation's norm preservation and relative-
position property, the identity at the origin, and a hand-computed rotation.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6
BASE = 10000.0


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def rms_norm(X, gamma, eps: float = EPS) -> np.ndarray:
    """x / sqrt(mean_c x_c^2 + eps) * gamma, per token over the last axis."""
    X = _f64(X)
    ms = np.mean(X * X, axis=-1, keepdims=True)
    return X / np.sqrt(ms + eps) * _f64(gamma)


def rope_bands(d: int) -> list[int]:
    """Channel counts of the (t, y, x) bands of a head of width d."""
    if d % 16:
        raise ValueError("head width must be a multiple of 16 (even bands)")
    return [d // 4, 3 * d // 8, 3 * d // 8]


def token_coords(F: int, Hg: int, Wg: int) -> np.ndarray:
    """(t, y, x) of every token of a chunk, frame-major: [F*Hg*Wg, 3]."""
    T = Hg * Wg
    n = np.arange(F * T)
    return np.stack([n // T, (n % T) // Wg, n % Wg], axis=1)


def rope_angles(coords, d: int, base: float = BASE) -> np.ndarray:
    """Angle of every channel pair of every token: [n_tokens, d/2]."""
    coords = np.asarray(coords)
    cols = []
    for band, n_b in enumerate(rope_bands(d)):
        i = np.arange(n_b // 2)
        freq = base ** (-2.0 * i / n_b)
        cols.append(coords[:, band:band + 1].astype(np.float64) * freq[None, :])
    return np.concatenate(cols, axis=1)


def apply_rope(U, angles) -> np.ndarray:
    """Turn channel pairs (2i, 2i+1) of U [..., n, d] by angles [n, d/2]."""
    U = _f64(U)
    c = np.cos(angles)
    s = np.sin(angles)
    a = U[..., 0::2]
    b = U[..., 1::2]
    out = np.empty_like(U)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def prep_rows(X, W, gamma, F: int, Hg: int, Wg: int, H: int, d: int, b: int, rows,
              eps: float = EPS, base: float = BASE):
    """Q, K, V [H, len(rows), d] of the tokens ``rows`` of batch b: every step
    of the chain is per token, so a subset of tokens is computed alone."""
    rows = np.asarray(rows, dtype=np.int64)
    C = H * d
    x = _f64(X[b][rows])
    y = rms_norm(x, gamma, eps) @ _f64(W).T                      # [n, 3C]
    ang = rope_angles(token_coords(F, Hg, Wg)[rows], d, base)
    def head(part, h):
        return y[:, part * C + h * d:part * C + (h + 1) * d]
    Q = np.stack([apply_rope(head(0, h), ang) for h in range(H)])
    K = np.stack([apply_rope(head(1, h), ang) for h in range(H)])
    V = np.stack([head(2, h) for h in range(H)])
    return Q, K, V


def prep(X, W, gamma, F: int, Hg: int, Wg: int, H: int, d: int,
         eps: float = EPS, base: float = BASE):
    """Q, K, V [B, H, N, d] (float64) from tokens X [B, N, C], C = H*d.

    RMSNorm, the joint projection, head packing, then the rotary embedding
    of queries and keys ("Layout Is the ABI" ¶2).
    """
    X = _f64(X)
    B, N, C = X.shape
    assert C == H * d and N == F * Hg * Wg
    out = [prep_rows(X, W, gamma, F, Hg, Wg, H, d, b, np.arange(N), eps, base)
           for b in range(B)]
    return tuple(np.stack([o[i] for o in out]) for i in range(3))
