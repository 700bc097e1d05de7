"""Pins of the fp64 oracle to facts other than itself (CPU only).

Each test ties an oracle function to a brute-force construction, a library
routine, a closed form or an exact invariant. The source page ("HeyGen 与
Google Cloud：将 Avatar IV 部署到 TPU", news.xcc.im/article/5328) prints no
worked example, so the only stored values are the hand-derived slice sizes in
tests/golden/.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import fsa_oracle as orc
from frame_aligned_block_amd.inputs import CONFIGS, make_cross_head, make_head, make_inputs, to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "slice_sizes.json")


def golden_cases():
    with open(GOLDEN) as fh:
        return json.load(fh)["cases"]


def dense_mask(F, T, window, ref_frame):
    """N x N boolean mask built element by element from the definition:
    key j is visible to query i iff the frames differ by at most the window,
    or key j lies in the reference frame."""
    fi = np.arange(F * T)[:, None] // T
    fj = np.arange(F * T)[None, :] // T
    return (np.abs(fi - fj) <= window) | (fj == ref_frame)


def rand_qkv(rng, B, H, N, d, mean_scale=0.0):
    Q = rng.standard_normal((B, H, N, d))
    K = rng.standard_normal((B, H, N, d)) + mean_scale * rng.standard_normal((B, H, 1, d))
    V = rng.standard_normal((B, H, N, d))
    return Q, K, V


# ---------------------------------------------------------------- slice / plan

@pytest.mark.parametrize("case", golden_cases(), ids=lambda c: c["name"])
def test_slice_sizes_match_hand_derivation(case):
    F, w, r = case["F"], case["window"], case["ref_frame"]
    sizes = [len(orc.slice_frames(F, w, r, f)) for f in range(F)]
    assert sizes == case["slice_sizes"]
    assert orc.valid_pairs_per_head(F, case["T"], w, r) == case["total"] * case["T"] ** 2


@pytest.mark.parametrize("case", golden_cases(), ids=lambda c: c["name"])
def test_plan_tile_count_closed_form(case):
    F, T, w, r = case["F"], case["T"], case["window"], case["ref_frame"]
    blocks = [b for b in range(16, T + 1, 16) if T % b == 0]
    for bq in blocks[:3]:
        for bk in blocks[-2:]:
            p = orc.plan(F, T, w, r, bq, bk)
            assert p["nnz"] == case["total"] * (T // bq) * (T // bk)


@pytest.mark.parametrize("F,T,w,r,bq,bk", [
    (5, 48, 1, 0, 16, 16), (5, 48, 1, 0, 48, 16), (5, 48, 1, 0, 16, 48),
    (7, 32, 1, 3, 16, 32), (6, 48, 0, 5, 48, 48), (4, 16, 3, 2, 16, 16),
    (9, 880, 2, 0, 80, 176), (9, 880, 2, 0, 880, 16),
])
def test_plan_matches_bruteforce_mask(F, T, w, r, bq, bk):
    mask = dense_mask(F, T, w, r)
    nqb, nkb = F * T // bq, F * T // bk
    tiles = mask.reshape(nqb, bq, nkb, bk)
    live = tiles.any(axis=(1, 3))
    full = tiles.all(axis=(1, 3))
    # frame alignment: a live tile is a full tile, never a partial one
    assert np.array_equal(live, full)
    p = orc.plan(F, T, w, r, bq, bk)
    ref_rows, ref_cols = np.nonzero(live)          # row-major: (qb asc, kb asc)
    assert np.array_equal(p["col_idx"], ref_cols)
    assert np.array_equal(p["row_ptr"], np.concatenate([[0], np.cumsum(live.sum(axis=1))]))
    assert np.array_equal(p["qframe"], np.arange(nqb) * bq // T)
    # runs cover exactly the live key tokens of each q-block, in order
    for qb in range(nqb):
        toks = np.concatenate([np.arange(a, e) for a, e in p["runs"][qb]])
        assert np.array_equal(toks, np.nonzero(mask[qb * bq])[0])
        assert len(p["runs"][qb]) <= 2


def test_plan_rejects_unaligned_blocks():
    with pytest.raises(ValueError):
        orc.plan(5, 48, 1, 0, 32, 16)       # 32 does not divide 48
    with pytest.raises(ValueError):
        orc.plan(5, 48, 1, 0, 24, 24)       # not a multiple of 16


# ---------------------------------------------------------------- attention

def loops_attention(Q, K, V, F, T, w, r, scale):
    """Masked softmax attention by explicit scalar loops (math.exp)."""
    N, d = Q.shape
    out = np.zeros((N, d))
    for i in range(N):
        fi = i // T
        js = [j for j in range(N) if abs(j // T - fi) <= w or j // T == r]
        s = [scale * sum(Q[i, c] * K[j, c] for c in range(d)) for j in js]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = sum(e)
        for c in range(d):
            out[i, c] = sum(e[n] * V[js[n], c] for n in range(len(js))) / z
    return out


@pytest.mark.parametrize("F,T,w,r", [(4, 16, 1, 2), (5, 16, 0, 0), (3, 16, 1, 0)])
def test_attention_matches_scalar_loops(F, T, w, r):
    rng = np.random.default_rng(11)
    d = 8
    Q, K, V = rand_qkv(rng, 1, 1, F * T, d)
    want = loops_attention(Q[0, 0], K[0, 0], V[0, 0], F, T, w, r, 0.37)
    got = orc.attention(Q, K, V, F, T, w, r, 0.37)[0, 0]
    assert np.max(np.abs(got - want)) < 1e-12


@pytest.mark.parametrize("F,T,w,r", [(5, 48, 1, 0), (7, 32, 1, 3), (6, 16, 2, 5), (4, 48, 3, 1)])
def test_attention_matches_torch_sdpa_with_mask(F, T, w, r):
    rng = np.random.default_rng(5)
    d = 64
    Q, K, V = rand_qkv(rng, 1, 2, F * T, d, mean_scale=3.0)
    scale = 1 / math.sqrt(d)
    mask = torch.from_numpy(dense_mask(F, T, w, r))
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V),
        attn_mask=mask, scale=scale).numpy()
    got = orc.attention(Q, K, V, F, T, w, r, scale)
    assert np.max(np.abs(got - want)) < 1e-12


def test_full_window_is_dense_attention():
    cfg = CONFIGS["tiny"]
    Q, K, V = (to_f64(t) for t in make_inputs(cfg, seed=3))
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V),
        scale=cfg.scale).numpy()
    got = orc.attention(Q, K, V, cfg.F, cfg.T, cfg.F - 1, 2, cfg.scale)
    assert np.max(np.abs(got - want)) < 1e-12


def test_attention_rows_matches_full():
    cfg = CONFIGS["tiny"]
    Q, K, V = (to_f64(t) for t in make_inputs(cfg))
    full = orc.attention(Q, K, V, cfg.F, cfg.T, cfg.window, cfg.ref_frame, cfg.scale)
    rows = np.array([0, 47, 48, 100, 239, 150])
    part = orc.attention_rows(Q, K, V, cfg.F, cfg.T, cfg.window, cfg.ref_frame,
                              cfg.scale, 0, 1, rows)
    assert np.max(np.abs(part - full[0, 1, rows])) < 1e-14


def test_centring_invariance():
    rng = np.random.default_rng(2)
    F, T, w, r, d = 6, 32, 1, 0, 32
    Q, K, V = rand_qkv(rng, 1, 2, F * T, d, mean_scale=4.0)
    base = orc.attention(Q, K, V, F, T, w, r, 0.2)
    mu = orc.key_mean(K)
    centred = orc.attention(Q, K - mu[:, :, None, :], V, F, T, w, r, 0.2)
    shifted = orc.attention(Q, K + rng.standard_normal((1, 2, 1, d)), V, F, T, w, r, 0.2)
    assert np.max(np.abs(centred - base)) < 1e-12
    assert np.max(np.abs(shifted - base)) < 1e-12


def test_key_mean_closed_form():
    # keys = c +/- a_j e_k in pairs: the mean is exactly c
    d, c = 8, np.arange(1.0, 9.0)
    dev = np.zeros((16, d))
    for j in range(8):
        dev[2 * j, j] = j + 0.5
        dev[2 * j + 1, j] = -(j + 0.5)
    K = (c + dev)[None, None]
    assert np.allclose(orc.key_mean(K)[0, 0], c, rtol=0, atol=1e-15)


# ---------------------------------------------------------------- bounds

def test_bounds_hand_case():
    """F=3 frames of T=16 tokens, d=4, window 0, reference frame 2.

    Keys are mu + x_j with mu = (1, -2, 3, 0.5) and deviations x_j that cancel
    over the chunk; frame g's largest deviation norm is 1, 5 and 2.
    Slices: frame 0 -> {0, 2}, frame 1 -> {1, 2}, frame 2 -> {2}; so
    R_S = (max(1,2), max(5,2), 2) = (2, 5, 2).
    Queries: row 3 of frame 0 is (3, 4, 0, 0) (norm 5), row 16+7 is
    (0, 0, 0, 2) (norm 2), row 32+1 is (1, 1, 1, 1) (norm 2); all other rows 0.
    With scale 0.5 the row bounds are 0.5*5*2 = 5, 0.5*2*5 = 5, 0.5*2*2 = 2,
    so stat = 5 (eligible); with scale 8 the stat is 80 (not eligible).
    """
    F, T, d = 3, 16, 4
    mu = np.array([1.0, -2.0, 3.0, 0.5])
    x = np.zeros((F * T, d))
    x[0] = [1, 0, 0, 0]; x[1] = [-1, 0, 0, 0]           # frame 0: norm 1
    x[16] = [0, 3, 4, 0]; x[17] = [0, -3, -4, 0]         # frame 1: norm 5
    x[18] = [0, 1, 0, 0]; x[19] = [0, -1, 0, 0]
    x[32] = [0, 0, 0, 2]; x[33] = [0, 0, 0, -2]          # frame 2: norm 2
    Q = np.zeros((F * T, d))
    Q[3] = [3, 4, 0, 0]; Q[23] = [0, 0, 0, 2]; Q[33] = [1, 1, 1, 1]
    K = (mu + x)[None, None]
    b = orc.bounds(Q[None, None], K, F, T, 0, 2, 0.5)
    assert np.allclose(b["mu"][0, 0], mu, atol=1e-15)
    assert np.allclose(b["R"][0, 0], [1, 5, 2], atol=1e-15)
    assert np.allclose(b["R_S"][0, 0], [2, 5, 2], atol=1e-15)
    assert np.allclose(b["qnorm"][0, 0, [3, 23, 33, 0]], [5, 2, 2, 0], atol=1e-15)
    assert np.allclose(b["bound"][0, 0, [3, 23, 33]], [5, 5, 2], atol=1e-15)
    assert b["stat"][0, 0] == pytest.approx(5.0, abs=1e-14)
    assert bool(b["elig"][0, 0])
    # the threshold is inclusive: the largest row bound is 10 * scale, and
    # scale 3.2 gives exactly 32.0 in fp64 (3.2*5 and 6.4*5 round to 16, 32)
    for scale, elig in [(2.0, True), (3.2, True), (3.25, False)]:
        bs = orc.bounds(Q[None, None], K, F, T, 0, 2, scale)
        assert bs["stat"][0, 0] == pytest.approx(10 * scale, abs=1e-12)
        assert bool(bs["elig"][0, 0]) == elig, scale
    b8 = orc.bounds(Q[None, None], K, F, T, 0, 2, 8.0)
    assert b8["stat"][0, 0] == pytest.approx(80.0, abs=1e-12)
    assert not bool(b8["elig"][0, 0])
    # without centring the norms are those of the raw keys
    raw = orc.bounds(Q[None, None], K, F, T, 0, 2, 0.5, centre=False)
    assert np.allclose(raw["R"][0, 0], np.linalg.norm(K[0, 0], axis=1).reshape(F, T).max(1))


def centred_logit_max(Q, K, F, T, w, r, scale, b, h, rows):
    mu = K[b, h].mean(axis=0)
    out = []
    for i in rows:
        keys = [j for j in range(F * T) if abs(j // T - i // T) <= w or j // T == r]
        out.append((scale * ((K[b, h][keys] - mu) @ Q[b, h][i])).max())
    return np.array(out)


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_bound_is_at_least_the_true_row_max(name):
    cfg = CONFIGS[name]
    rng = np.random.default_rng(1)
    q, k, v = make_head(cfg, 0, 0, 0)
    Q, K = to_f64(q)[None, None], to_f64(k)[None, None]
    bnd = orc.bounds(Q, K, cfg.F, cfg.T, cfg.window, cfg.ref_frame, cfg.scale)
    rows = np.arange(cfg.N) if name == "tiny" else rng.choice(cfg.N, 300, replace=False)
    m = centred_logit_max(Q, K, cfg.F, cfg.T, cfg.window, cfg.ref_frame, cfg.scale, 0, 0, rows)
    assert np.all(bnd["bound"][0, 0, rows] >= m)
    # and the bound is not vacuous: the gap stays well below the bound itself
    assert np.median(bnd["bound"][0, 0, rows] - m) < np.median(bnd["bound"][0, 0, rows])


def test_bound_is_attained_when_query_parallel_to_the_longest_key():
    rng = np.random.default_rng(4)
    F, T, d = 3, 16, 16
    Q, K, _ = rand_qkv(rng, 1, 1, F * T, d, mean_scale=2.0)
    kc = K[0, 0] - K[0, 0].mean(axis=0)
    j = int(np.argmax(np.linalg.norm(kc, axis=1)))
    Q[0, 0, 5] = 0.7 * kc[j]                        # row 5 sits in frame 0
    bnd = orc.bounds(Q, K, F, T, 2, 0, 0.25)       # window covers every frame
    s = 0.25 * (kc @ Q[0, 0, 5])
    assert bnd["bound"][0, 0, 5] == pytest.approx(s.max(), rel=1e-14)


def test_eligibility_by_construction_on_full_size_heads():
    """Normal heads of the full-size configs are eligible with a margin; the
    stress config's loose head (h % 50 == 7) is not; without centring the
    normal heads would not be eligible (centring tightens the bound)."""
    margin = 1.05
    for name, h in [("720p", 0), ("1080p", 3), ("stress", 6), ("stress", 7), ("720p-dense", 0)]:
        cfg = CONFIGS[name]
        q, k, _ = make_head(cfg, 0, 0, h)
        Q, K = to_f64(q)[None, None], to_f64(k)[None, None]
        b = orc.bounds(Q, K, cfg.F, cfg.T, cfg.window, cfg.ref_frame, cfg.scale)
        stat = b["stat"][0, 0]
        if cfg.is_loose(h):
            assert stat > orc.BETA * margin, (name, h, stat)
            assert not bool(b["elig"][0, 0])
        else:
            assert stat < orc.BETA / margin, (name, h, stat)
            assert bool(b["elig"][0, 0])
            raw = orc.bounds(Q, K, cfg.F, cfg.T, cfg.window, cfg.ref_frame,
                             cfg.scale, centre=False)
            assert raw["stat"][0, 0] > orc.BETA * margin, (name, h, raw["stat"])


def test_frame_eligibility_follows_the_outlier_frame():
    """Per (head, frame) eligibility on the outlier-frame workload: a loose
    head's outlier keys sit in frame 6 only, so exactly the frames whose slice
    (window +-2, reference frame 0) holds frame 6 fail, by a wide margin, and
    every other frame passes, as do all frames of a normal head; the head-level
    flag is their conjunction."""
    cfg = CONFIGS["outlier-frame"]
    margin = 1.05
    for h in (0, 1):
        q, k, _ = make_head(cfg, 0, 0, h)
        Q, K = to_f64(q)[None, None], to_f64(k)[None, None]
        b = orc.bounds(Q, K, cfg.F, cfg.T, cfg.window, cfg.ref_frame, cfg.scale)
        sees_outlier = [6 in orc.slice_frames(cfg.F, cfg.window, cfg.ref_frame, f)
                        for f in range(cfg.F)]
        assert sees_outlier == [f in (4, 5, 6, 7, 8) for f in range(cfg.F)]
        for f in range(cfg.F):
            sf = b["stat_frame"][0, 0, f]
            if cfg.is_loose(h) and sees_outlier[f]:
                assert sf > orc.BETA * margin and not b["elig_frame"][0, 0, f], (h, f, sf)
            else:
                assert sf < orc.BETA / margin and b["elig_frame"][0, 0, f], (h, f, sf)
        assert b["stat"][0, 0] == b["stat_frame"][0, 0].max()
        assert bool(b["elig"][0, 0]) == bool(b["elig_frame"][0, 0].all())


# ---------------------------------------------------------------- gap bound

def test_gap_bound_hand_case():
    """A case small enough to work out on paper (d = 2, scale 1, F = 2 frames
    of T = 2 tokens, window 0, reference frame 0, so S(0) = {0} and
    S(1) = {0, 1}). Keys: frame 0 (1,0), (3,0); frame 1 (-1,0), (-3,0); their
    mean is 0, every frame's largest norm is 3, the slice means are (2,0) and
    (0,0). Rows q = (1,0), (-1,0) in frame 0 and (1,0), (0,2) in frame 1 have
    bounds 3, 3, 3, 6 and gap bounds 3-2 = 1, 3+2 = 5, 3, 6. Their true gaps
    (bound minus the largest logit) are 0, 4, 0 and 6: the last row scores
    every key 0, so its bound is tight."""
    K = np.array([[1.0, 0.0], [3.0, 0.0], [-1.0, 0.0], [-3.0, 0.0]])[None, None]
    Q = np.array([[1.0, 0.0], [-1.0, 0.0], [1.0, 0.0], [0.0, 2.0]])[None, None]
    g = orc.gap_bounds(Q, K, 2, 2, 0, 0, 1.0)
    assert np.allclose(g["bound"][0, 0], [3, 3, 3, 6], rtol=0, atol=1e-15)
    assert np.allclose(g["gap"][0, 0], [1, 5, 3, 6], rtol=0, atol=1e-15)
    assert np.allclose(g["dslice"][0, 0], [[2, 0], [0, 0]], rtol=0, atol=1e-15)
    true_gap = np.array([3 - 3, 3 - (-1), 3 - 3, 6 - 0])
    assert np.all(g["gap"][0, 0] >= true_gap)
    assert g["ok"][0, 0].all() and not orc.gap_bounds(Q, K, 2, 2, 0, 0, 1.0, limit=5.5)["ok"][0, 0, 3]


@pytest.mark.parametrize("name", ["tiny", "loose-rows-small", "stress"])
def test_gap_bound_brackets_the_true_gap(name):
    """For every row (sampled rows at the 720p shape), brute force in fp64:
    B_i - max_j scale <q_i, k_j - mu> <= G_i <= 2 B_i, the upper end by
    Cauchy-Schwarz on the slice mean. Head 7 of stress is its loose head."""
    cfg = CONFIGS[name]
    h = 7 if name == "stress" else 1
    q, k, _ = make_head(cfg, 0, 0, h)
    Q, K = to_f64(q)[None, None], to_f64(k)[None, None]
    g = orc.gap_bounds(Q, K, cfg.F, cfg.T, cfg.window, cfg.ref_frame, cfg.scale)
    rng = np.random.default_rng(3)
    rows = np.arange(cfg.N) if cfg.N <= 5000 else rng.choice(cfg.N, 400, replace=False)
    mu = K[0, 0].mean(axis=0)
    for i in rows:
        keys = orc.slice_keys(cfg.F, cfg.T, cfg.window, cfg.ref_frame, int(i) // cfg.T)
        true_max = (cfg.scale * ((K[0, 0, keys] - mu) @ Q[0, 0, i])).max()
        true_gap = g["bound"][0, 0, i] - true_max
        assert true_gap <= g["gap"][0, 0, i] * (1 + 1e-12) + 1e-12, (i, true_gap, g["gap"][0, 0, i])
        assert g["gap"][0, 0, i] <= 2 * g["bound"][0, 0, i] * (1 + 1e-12), i


def test_gap_bound_invariances():
    """Moving every key by one vector changes neither the slice offsets nor the
    gap bounds (they are taken from centred keys); a window that covers every
    frame makes each slice the whole chunk, whose mean is mu, so G_i = B_i."""
    rng = np.random.default_rng(5)
    F, T, d = 5, 16, 8
    Q, K, _ = rand_qkv(rng, 1, 2, F * T, d, mean_scale=2.0)
    a = orc.gap_bounds(Q, K, F, T, 1, 0, 0.4)
    b = orc.gap_bounds(Q, K + rng.standard_normal((1, 2, 1, d)) * 5.0, F, T, 1, 0, 0.4)
    assert np.allclose(a["gap"], b["gap"], rtol=1e-12, atol=1e-12)
    assert np.allclose(a["dslice"], b["dslice"], rtol=1e-12, atol=1e-12)
    full = orc.gap_bounds(Q, K, F, T, F - 1, 0, 0.4)
    assert np.allclose(full["dslice"], 0.0, atol=1e-13)
    assert np.allclose(full["gap"], full["bound"], rtol=1e-13)


@pytest.mark.parametrize("name", ["loose-rows-small", "loose-rows"])
def test_gap_rows_by_construction(name):
    """The looser workloads: every head's largest bound is far above BETA (the
    per-head and per-frame checks fail everywhere), yet every row outside a
    frame's hot band has a gap bound well within GAP_LIMIT, and every frame's
    hot band holds rows well beyond it."""
    cfg = CONFIGS[name]
    margin = 1.05
    for h in (0, 2):
        q, k, _ = make_head(cfg, 0, 0, h)
        Q, K = to_f64(q)[None, None], to_f64(k)[None, None]
        b = orc.bounds(Q, K, cfg.F, cfg.T, cfg.window, cfg.ref_frame, cfg.scale)
        assert (b["stat_frame"][0, 0] > orc.BETA * margin).all(), h
        g = orc.gap_bounds(Q, K, cfg.F, cfg.T, cfg.window, cfg.ref_frame, cfg.scale)
        qn = b["qnorm"][0, 0].reshape(cfg.F, cfg.T)
        gap = g["gap"][0, 0].reshape(cfg.F, cfg.T)
        for f in range(cfg.F):
            # the band is where the norms are scaled: a contiguous run of hot_rows
            med = np.median(qn[f])
            hot = qn[f] > 1.6 * med
            idx = np.flatnonzero(hot)
            assert len(idx) > 0.9 * cfg.hot_rows and idx[-1] - idx[0] < cfg.hot_rows, (h, f)
            assert gap[f, ~hot].max() < orc.GAP_LIMIT / 1.5, (h, f)
            assert gap[f, hot].max() > orc.GAP_LIMIT * margin, (h, f)


def test_cross_gap_bound_is_the_bound():
    """Cross-attention: every row's slice is the whole reference set, so the
    slice mean is mu and the gap bound equals the bound; it still brackets the
    true gap (brute force)."""
    rng = np.random.default_rng(9)
    F, T, M, d = 3, 16, 24, 8
    Q = rng.standard_normal((1, 1, F * T, d))
    Kr = rng.standard_normal((1, 1, M, d)) + 2.0
    b = orc.cross_bounds(Q, Kr, F, T, 0.5)
    assert np.array_equal(b["gap"], b["bound"])
    kc = Kr[0, 0] - Kr[0, 0].mean(axis=0)
    true_gap = b["bound"][0, 0] - (0.5 * (Q[0, 0] @ kc.T)).max(axis=1)
    assert np.all(true_gap <= b["gap"][0, 0] + 1e-12)


# ---------------------------------------------------------------- routes

def test_fixed_max_and_online_routes_equal_the_definition():
    cfg = CONFIGS["small"]
    q, k, v = make_head(cfg, 0, 0, 5)
    Q, K, V = (to_f64(t)[None, None] for t in (q, k, v))
    rng = np.random.default_rng(9)
    rows = np.sort(rng.choice(cfg.N, 40, replace=False))
    args = (Q, K, V, cfg.F, cfg.T, cfg.window, cfg.ref_frame, cfg.scale, 0, 0, rows)
    want = orc.attention_rows(*args)
    assert np.max(np.abs(orc.attention_fixed_max(*args) - want)) < 1e-12
    assert np.max(np.abs(orc.attention_online(*args, block=80) - want)) < 1e-12
    assert np.max(np.abs(orc.attention_online(*args, block=16, centre=False) - want)) < 1e-12


def test_two_pass_merge_equals_single_pass_and_pins_no_double_count():
    F, T, w, d = 7, 16, 1, 16
    rng = np.random.default_rng(8)
    Q, K, V = rand_qkv(rng, 1, 1, F * T, d)
    r = 3
    rows = np.arange(F * T)
    want = orc.attention_rows(Q, K, V, F, T, w, r, 0.3, 0, 0, rows)
    got = orc.attention_two_pass(Q, K, V, F, T, w, r, 0.3, 0, 0, rows)
    assert np.max(np.abs(got - want)) < 1e-12
    # rows of frames 2..4 hold the reference frame in their window already:
    inside = rows[(rows // T >= 2) & (rows // T <= 4)]
    dbl = orc.attention_two_pass(Q, K, V, F, T, w, r, 0.3, 0, 0, inside, add_ref_always=True)
    assert np.min(np.max(np.abs(dbl - want[inside]), axis=1)) > 1e-6


# ---------------------------------------------------------------- probes

def test_structured_value_probes():
    F, T, w, r, d = 6, 32, 1, 4, 16
    N = F * T
    rng = np.random.default_rng(6)
    Q, K, _ = rand_qkv(rng, 1, 1, N, d, mean_scale=2.0)
    frame = np.arange(N) // T
    # (i) one-hot frame values: weight lands only on the slice's frames
    V1 = np.zeros((1, 1, N, d))
    V1[0, 0, np.arange(N), frame] = 1.0
    O = orc.attention(Q, K, V1, F, T, w, r, 0.5)[0, 0]
    for i in range(N):
        allowed = {g for g in range(F) if abs(g - i // T) <= w} | {r}
        for g in range(F):
            if g not in allowed:
                assert O[i, g] == 0.0
        assert abs(O[i, :F].sum() - 1.0) < 1e-12
    # (ii) one-hot 16-key granule values: every granule of the slice gets weight
    V2 = np.zeros((1, 1, N, d))
    V2[0, 0, np.arange(N), (np.arange(N) // 16) % d] = 1.0
    O2 = orc.attention(Q, K, V2, F, T, w, r, 0.5)[0, 0]
    assert np.all(np.abs(O2.sum(axis=1) - 1.0) < 1e-12)
    # (iii) constant values pass through exactly
    O3 = orc.attention(Q, K, np.ones((1, 1, N, d)), F, T, w, r, 0.5)
    assert np.max(np.abs(O3 - 1.0)) < 1e-14
    # (iv) zero queries give the plain mean of the slice's values
    V4 = rng.standard_normal((1, 1, N, d))
    O4 = orc.attention(np.zeros((1, 1, N, d)), K, V4, F, T, w, r, 0.5)[0, 0]
    for f in range(F):
        sel = (np.abs(frame - f) <= w) | (frame == r)
        want = V4[0, 0][sel].mean(axis=0)
        assert np.max(np.abs(O4[f * T:(f + 1) * T] - want)) < 1e-13


# ---------------------------------------------------------------- cross-attention

def test_cross_attention_matches_torch_sdpa():
    rng = np.random.default_rng(11)
    B, H, N, M, d = 1, 2, 96, 48, 32
    Q = rng.standard_normal((B, H, N, d))
    Kr = rng.standard_normal((B, H, M, d)) + 3.0 * rng.standard_normal((B, H, 1, d))
    Vr = rng.standard_normal((B, H, M, d))
    scale = 1 / math.sqrt(d)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q), torch.from_numpy(Kr), torch.from_numpy(Vr), scale=scale).numpy()
    assert np.max(np.abs(orc.cross_attention(Q, Kr, Vr, scale) - want)) < 1e-12
    rows = np.array([0, 5, 95, 40])
    part = orc.cross_attention_rows(Q, Kr, Vr, scale, 0, 1, rows)
    assert np.max(np.abs(part - want[0, 1, rows])) < 1e-12


def test_cross_attention_invariances_and_bound():
    """A shared offset on every reference key leaves the output unchanged
    (each row's logits move together); constant values pass through; the
    bound of every row is at least its largest centred logit, and is reached
    when the query is parallel to the longest centred key."""
    rng = np.random.default_rng(12)
    F, T, M, d = 3, 16, 32, 16
    N = F * T
    Q = rng.standard_normal((1, 1, N, d))
    Kr = rng.standard_normal((1, 1, M, d))
    Vr = rng.standard_normal((1, 1, M, d))
    base = orc.cross_attention(Q, Kr, Vr, 0.3)
    shifted = orc.cross_attention(Q, Kr + 5.0 * rng.standard_normal((1, 1, 1, d)), Vr, 0.3)
    assert np.max(np.abs(base - shifted)) < 1e-12
    ones = orc.cross_attention(Q, Kr, np.ones((1, 1, M, d)), 0.3)
    assert np.max(np.abs(ones - 1.0)) < 1e-14
    b = orc.cross_bounds(Q, Kr, F, T, 0.3)
    kc = Kr[0, 0] - Kr[0, 0].mean(axis=0)
    logits = 0.3 * (Q[0, 0] @ kc.T)
    assert np.all(b["bound"][0, 0] >= logits.max(axis=1) - 1e-12)
    j = int(np.argmax(np.linalg.norm(kc, axis=1)))
    Q2 = Q.copy()
    Q2[0, 0, 7] = 0.5 * kc[j]
    b2 = orc.cross_bounds(Q2, Kr, F, T, 0.3)
    assert b2["bound"][0, 0, 7] == pytest.approx((0.3 * (Q2[0, 0, 7] @ kc.T)).max(), rel=1e-13)
    assert b["stat"][0, 0] == b["stat_frame"][0, 0].max()


def test_cross_eligibility_by_construction():
    """A normal cross head (reference keys with a shared mean) is eligible once
    centred and not without centring; the small cross workload's head 3, with
    one reference key scaled by 20, is not."""
    margin = 1.05
    for name, h in [("720p-xref", 0), ("xref-small", 0), ("xref-small", 3)]:
        cfg = CONFIGS[name]
        q, k, _ = make_cross_head(cfg, 0, 0, h)
        Q, K = to_f64(q)[None, None], to_f64(k)[None, None]
        b = orc.cross_bounds(Q, K, cfg.F, cfg.T, cfg.scale)
        stat = b["stat"][0, 0]
        if cfg.is_loose(h):
            assert stat > orc.BETA * margin and not b["elig"][0, 0], (name, h, stat)
        else:
            assert stat < orc.BETA / margin and b["elig"][0, 0], (name, h, stat)
            raw = cfg.scale * np.linalg.norm(Q[0, 0], axis=1).max() * np.linalg.norm(K[0, 0], axis=1).max()
            assert raw > orc.BETA * margin, (name, h, raw)


@pytest.mark.parametrize("F,T,M,bq,bk", [(3, 48, 80, 16, 16), (4, 96, 48, 32, 48),
                                         (2, 160, 320, 80, 64), (5, 16, 16, 16, 16)])
def test_cross_plan_against_bruteforce_tiles_and_closed_forms(F, T, M, bq, bk):
    """cross_plan against the definition written out pair by pair: a tile is
    live iff some (query, reference key) pair in it attends, and in
    cross-attention every pair does, so the live set is the full grid of
    (F*T/bq) x (M/bk) tiles; each q-block's frame is floor(qb*bq / T) and its
    one key run is the whole set [0, M)."""
    p = orc.cross_plan(F, T, M, bq, bk)
    nqb, nkb = F * T // bq, M // bk
    live = np.zeros((nqb, nkb), dtype=bool)
    for i in range(F * T):              # brute force over every pair
        for j in range(M):
            live[i // bq, j // bk] = True
    rows, cols = np.nonzero(live)        # row-major: ascending qb, then kb
    assert p["nnz"] == rows.size == nqb * nkb
    assert np.array_equal(p["col_idx"], cols)
    assert np.array_equal(p["row_ptr"], np.searchsorted(rows, np.arange(nqb + 1)))
    assert np.array_equal(p["qframe"], [(qb * bq) // T for qb in range(nqb)])
    assert p["runs"] == [[(0, M)]] * nqb


@pytest.mark.parametrize("F,T,bq,bk", [(3, 48, 16, 48), (4, 32, 32, 16), (2, 96, 48, 32)])
def test_cross_plan_equals_the_dense_self_plan(F, T, bq, bk):
    """Two independent routes to one tile list: cross-attention to a reference
    set of M = F*T keys and self-attention whose window covers every frame both
    make every tile live, so their CSR arrays and q-block frames agree."""
    c = orc.cross_plan(F, T, F * T, bq, bk)
    s = orc.plan(F, T, F - 1, 0, bq, bk)
    for k in ("row_ptr", "col_idx", "qframe"):
        assert np.array_equal(np.asarray(c[k]), np.asarray(s[k])), k
