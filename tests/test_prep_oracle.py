"""Pins of the producer oracle (oracle/prep_oracle.py) to facts other than
itself (CPU only): torch's rms_norm and linear in float64, explicit loops, the
rotation's norm preservation and relative-position property, the identity at
the origin, and a rotation worked by hand."""
import math

import numpy as np
import pytest
import torch

from oracle import fsa_oracle as orc
from oracle import prep_oracle as prp
from frame_aligned_block_amd.inputs import CONFIGS, make_prep_inputs, to_f64


def test_rms_norm_matches_torch():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((2, 7, 48)) * 3.0 + 0.5
    g = 1.0 + 0.1 * rng.standard_normal(48)
    want = torch.nn.functional.rms_norm(torch.from_numpy(X), (48,), torch.from_numpy(g),
                                        eps=prp.EPS).numpy()
    assert np.max(np.abs(prp.rms_norm(X, g) - want)) < 1e-12


def test_rms_norm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((5, 64)) * 7.0
    Y = prp.rms_norm(X, np.ones(64), eps=0.0)
    assert np.allclose(np.sqrt(np.mean(Y * Y, axis=-1)), 1.0, atol=1e-12)
    assert np.allclose(prp.rms_norm(3.7 * X, np.ones(64), eps=0.0), Y, atol=1e-12)


def test_rope_bands():
    assert prp.rope_bands(128) == [32, 48, 48]
    assert prp.rope_bands(64) == [16, 24, 24]
    with pytest.raises(ValueError):
        prp.rope_bands(40)


def test_token_coords_frame_major():
    c = prp.token_coords(3, 2, 5)
    assert c.shape == (30, 3)
    assert list(c[0]) == [0, 0, 0] and list(c[4]) == [0, 0, 4] and list(c[5]) == [0, 1, 0]
    assert list(c[10]) == [1, 0, 0] and list(c[29]) == [2, 1, 4]


def test_rope_hand_case():
    """d = 16: bands of 4 (t), 6 (y), 6 (x) channels. At position (1, 0, 0)
    only the t band turns: pair 0 by 1 rad, pair 1 by 10000^(-1/2) = 0.01 rad."""
    u = np.arange(1.0, 17.0)[None, :]
    ang = prp.rope_angles(np.array([[1, 0, 0]]), 16)
    assert ang.shape == (1, 8)
    assert ang[0, 0] == 1.0 and abs(ang[0, 1] - 0.01) < 1e-15 and np.all(ang[0, 2:] == 0)
    out = prp.apply_rope(u, ang)[0]
    c1, s1, c2, s2 = math.cos(1.0), math.sin(1.0), math.cos(0.01), math.sin(0.01)
    assert abs(out[0] - (1 * c1 - 2 * s1)) < 1e-15 and abs(out[1] - (1 * s1 + 2 * c1)) < 1e-15
    assert abs(out[2] - (3 * c2 - 4 * s2)) < 1e-15 and abs(out[3] - (3 * s2 + 4 * c2)) < 1e-15
    assert np.array_equal(out[4:], u[0, 4:])
    # position (0, 2, 3): the y band's first pair turns by 2 rad, the x band's by 3
    ang = prp.rope_angles(np.array([[0, 2, 3]]), 16)
    out = prp.apply_rope(u, ang)[0]
    assert np.array_equal(out[:4], u[0, :4])
    assert abs(out[4] - (5 * math.cos(2) - 6 * math.sin(2))) < 1e-14
    assert abs(out[10] - (11 * math.cos(3) - 12 * math.sin(3))) < 1e-14


def test_rope_is_a_rotation_with_relative_positions():
    rng = np.random.default_rng(2)
    d = 128
    coords = prp.token_coords(5, 6, 7)
    q = rng.standard_normal((coords.shape[0], d))
    k = rng.standard_normal((coords.shape[0], d))
    ang = prp.rope_angles(coords, d)
    rq, rk = prp.apply_rope(q, ang), prp.apply_rope(k, ang)
    # norms preserved
    assert np.allclose(np.linalg.norm(rq, axis=1), np.linalg.norm(q, axis=1), rtol=1e-13)
    # the origin is the identity
    assert np.allclose(rq[0], q[0], atol=0) and np.allclose(rk[0], k[0], atol=0)
    # <R(q, P), R(k, P')> depends only on P - P': shift every position by (2, 3, 1)
    shifted = prp.rope_angles(coords + np.array([2, 3, 1]), d)
    sq, sk = prp.apply_rope(q, shifted), prp.apply_rope(k, shifted)
    assert np.allclose(rq @ rk.T, sq @ sk.T, atol=1e-10)
    # and it does depend on the offset: positions (0,0,0) vs (0,0,1) change the score
    assert abs(rq[0] @ rk[1] - q[0] @ k[1]) > 1e-3


def test_prep_matches_loops_on_a_tiny_case():
    rng = np.random.default_rng(3)
    F, Hg, Wg, H, d = 2, 1, 2, 2, 16
    C, N = H * d, F * Hg * Wg
    X = rng.standard_normal((1, N, C))
    W = rng.standard_normal((3 * C, C)) / math.sqrt(C)
    g = 1.0 + 0.1 * rng.standard_normal(C)
    Q, K, V = prp.prep(X, W, g, F, Hg, Wg, H, d)
    coords = prp.token_coords(F, Hg, Wg)
    for n in range(N):
        ms = sum(X[0, n, c] ** 2 for c in range(C)) / C
        xh = [X[0, n, c] / math.sqrt(ms + prp.EPS) * g[c] for c in range(C)]
        y = [sum(W[o, c] * xh[c] for c in range(C)) for o in range(3 * C)]
        t, yy, xx = coords[n]
        for h in range(H):
            for part, out in enumerate((Q, K, V)):
                u = [y[part * C + h * d + e] for e in range(d)]
                if part < 2:
                    start = 0
                    for n_b, p in zip(prp.rope_bands(d), (t, yy, xx)):
                        for i in range(n_b // 2):
                            th = p * prp.BASE ** (-2.0 * i / n_b)
                            a, b = u[start + 2 * i], u[start + 2 * i + 1]
                            u[start + 2 * i] = a * math.cos(th) - b * math.sin(th)
                            u[start + 2 * i + 1] = a * math.sin(th) + b * math.cos(th)
                        start += n_b
                assert np.allclose(out[0, h, n], u, atol=1e-12), (n, h, part)


def test_prep_matches_torch_composition():
    """RMSNorm and the projection through torch's own routines (float64); the
    values are the unrotated projection, and rotation is undone by the
    inverse angles."""
    rng = np.random.default_rng(4)
    F, Hg, Wg, H, d = 3, 4, 5, 2, 32
    C, N = H * d, F * Hg * Wg
    X = rng.standard_normal((2, N, C)) + 0.3
    W = rng.standard_normal((3 * C, C)) / math.sqrt(C)
    g = 1.0 + 0.1 * rng.standard_normal(C)
    Q, K, V = prp.prep(X, W, g, F, Hg, Wg, H, d)
    xt = torch.from_numpy(X)
    y = torch.nn.functional.linear(
        torch.nn.functional.rms_norm(xt, (C,), torch.from_numpy(g), eps=prp.EPS),
        torch.from_numpy(W)).numpy()
    heads = lambda part: y[:, :, part * C:(part + 1) * C].reshape(2, N, H, d).transpose(0, 2, 1, 3)
    assert np.allclose(V, heads(2), atol=1e-12)
    ang = prp.rope_angles(prp.token_coords(F, Hg, Wg), d)
    assert np.allclose(prp.apply_rope(Q, -ang), heads(0), atol=1e-12)
    assert np.allclose(prp.apply_rope(K, -ang), heads(1), atol=1e-12)


@pytest.mark.slow
def test_prep_workload_heads_are_eligible():
    """Every head of the small producer workload is eligible for the fixed
    max, clear of the threshold by 20%. (The rotation turns the keys' shared
    component by position-dependent angles, so centring tightens these
    bounds far less than the attention workloads' unrotated keys: about 1.2x.)"""
    cfg = CONFIGS["prep-small"]
    X, W, g = make_prep_inputs(cfg, seed=0)
    Hg, Wg = cfg.grid
    Q, K, _ = prp.prep(to_f64(X), to_f64(W), g.double().numpy(), cfg.F, Hg, Wg, cfg.H, cfg.d)
    b = orc.bounds(Q, K, cfg.F, cfg.T, cfg.window, cfg.ref_frame, cfg.scale)
    assert np.all(b["stat"] < 0.8 * orc.BETA), b["stat"]
    raw = orc.bounds(Q, K, cfg.F, cfg.T, cfg.window, cfg.ref_frame, cfg.scale, centre=False)
    assert np.all(raw["stat"] > b["stat"])
