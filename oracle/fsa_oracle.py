"""fp64 CPU oracle for frame-aligned windowed sparse attention.

TEST INFRASTRUCTURE. Only the tests, the package's smoke() check and the
benchmark's cpu_baseline leg may import or call this module. The product path
(the HIP library and its binding) never does, and this module imports nothing
from the product.

Source: the page "HeyGen 与 Google Cloud：将 Avatar IV 部署到 TPU"
(news.xcc.im/article/5328), English text; citations below name its section and
paragraph (figure captions are not counted as paragraphs).

What is computed (the definition; frame alignment, key centring and the fixed
max only change the route to it, never the exact result):
  * tokens are frame-major, token i lies in frame f(i) = i // T
    ("Hiding the Collective" ¶2: the mask is defined over a token ordering);
  * the key slice of frame f is S(f) = {g : 0 <= g < F, |g - f| <= w} U {r}:
    a window of neighbouring frames plus one global reference frame
    ("Deleting the Mask" ¶1);
  * O_i = sum_j exp(s_ij - m_i) v_j / sum_j exp(s_ij - m_i) over keys j whose
    frame is in S(f(i)), s_ij = scale * <q_i, k_j>, m_i = max_j s_ij.

Readings of points the page leaves open (each is listed in the design notes):
  * the window is clipped at the chunk edges, not shifted;
  * the reference frame joins the slice as a set union (counted once);
  * only query rows are frame-windowed: the reference frame's own queries see
    their own slice, not every key;
  * no causal masking inside a frame;
  * the key mean is one vector per (batch, head), over all N keys;
  * eligibility of a head: max over its rows of the Cauchy-Schwarz bound
    scale * ||q_i|| * max_{j in slice} ||k_j - mu|| is at most BETA = 32;
  * the finer, tighter check per row: the fixed max exceeds the row's true
    maximum by at most the gap bound G_i = B_i - scale <q_i, mean_S(k) - mu>
    (a maximum is at least the mean), and a row may take the fixed max when
    G_i <= GAP_LIMIT = 2 * BETA, the largest gap the per-head check allows.

Precision: every function upcasts its inputs to float64 and computes in
float64 with numpy; matrix products are numpy's.

Pins (tests that tie this module to facts other than itself): brute-force
masks and explicit loops, torch's scaled_dot_product_attention on the CPU in
float64, centring invariance, the bound against the true row max, closed-form
slice sizes and structured value probes. No function here is parity
unpinned. The cross-attention functions at the end are pinned the same way:
torch's scaled_dot_product_attention, invariance to a shared key offset,
constant values, and the bound against the true row max.
"""
from __future__ import annotations

import numpy as np

# Threshold on the per-head bound statistic (logit units). A head whose largest
# per-row bound exceeds it uses the online softmax path.
BETA = 32.0

# Limit on a row's gap bound (logit units): the per-head check bounds the gap
# by 2 * BETA (the logits of a row lie within +-B_i), so a row whose own gap
# bound is at most this keeps the same guarantee.
GAP_LIMIT = 2.0 * BETA

# Query rows processed together in one numpy product (memory bound, not math).
ROW_CHUNK = 512


# --------------------------------------------------------------------------
# the slice and the block plan  ("Deleting the Mask" ¶1-¶2)
# --------------------------------------------------------------------------

def slice_frames(F: int, window: int, ref_frame: int, f: int) -> list[int]:
    """Frames whose keys a query of frame f attends to, ascending.

    A window of up to ``window`` frames on each side of f, clipped to the
    chunk, joined with the reference frame ("Deleting the Mask" ¶1).
    """
    lo = max(0, f - window)
    hi = min(F - 1, f + window)
    frames = set(range(lo, hi + 1))
    frames.add(ref_frame)
    return sorted(frames)


def slice_keys(F: int, T: int, window: int, ref_frame: int, f: int) -> np.ndarray:
    """Token indices of frame f's key slice, ascending."""
    return np.concatenate([np.arange(g * T, (g + 1) * T)
                           for g in slice_frames(F, window, ref_frame, f)])


def valid_pairs_per_head(F: int, T: int, window: int, ref_frame: int) -> int:
    """Number of (query, key) pairs that attend, for one (batch, head)."""
    return sum(T * T * len(slice_frames(F, window, ref_frame, f)) for f in range(F))


def plan(F: int, T: int, window: int, ref_frame: int, bq: int, bk: int) -> dict:
    """Frame-aligned list of live (q-block, k-block) tiles in CSR form.

    Blocks are multiples of 16 tokens that divide the frame span, so no block
    straddles two frames and every tile is entirely inside or entirely outside
    the mask ("Deleting the Mask" ¶2). A tile is live iff its key block's frame
    is in the slice of its query block's frame. Rows are q-blocks in ascending
    order; each row lists its live k-blocks in ascending order.

    Also returns, per q-block, its live k-blocks merged into maximal runs of
    consecutive blocks, as token ranges [start, end).
    """
    if bq % 16 or bk % 16 or T % bq or T % bk:
        raise ValueError("block sizes must be multiples of 16 dividing T")
    nqb = F * T // bq
    nkb = F * T // bk
    row_ptr = [0]
    col_idx = []
    qframe = []
    runs = []
    for qb in range(nqb):
        f = qb * bq // T
        live_frames = set(slice_frames(F, window, ref_frame, f))
        cols = [kb for kb in range(nkb) if (kb * bk // T) in live_frames]
        col_idx.extend(cols)
        row_ptr.append(len(col_idx))
        qframe.append(f)
        row_runs = []
        for kb in cols:
            if row_runs and row_runs[-1][1] == kb * bk:
                row_runs[-1][1] = (kb + 1) * bk
            else:
                row_runs.append([kb * bk, (kb + 1) * bk])
        runs.append([tuple(r) for r in row_runs])
    return {
        "row_ptr": np.asarray(row_ptr, dtype=np.int64),
        "col_idx": np.asarray(col_idx, dtype=np.int64),
        "qframe": np.asarray(qframe, dtype=np.int64),
        "runs": runs,
        "nnz": len(col_idx),
    }


# --------------------------------------------------------------------------
# bounds  ("Unchaining the Softmax" ¶2-¶3)
# --------------------------------------------------------------------------

def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def key_mean(K) -> np.ndarray:
    """Mean of the keys over all N tokens, per (batch, head): [B, H, d]."""
    return _f64(K).mean(axis=-2)


def bounds(Q, K, F: int, T: int, window: int, ref_frame: int, scale: float,
           beta: float = BETA, centre: bool = True) -> dict:
    """Per-row Cauchy-Schwarz bounds and per-head eligibility.

    With keys centred by their mean mu (softmax-invariant, and tighter because
    the keys share a large common part; "Unchaining the Softmax" ¶2), the
    logit of row i against any key j of its slice satisfies
        |scale <q_i, k_j - mu>| <= scale ||q_i|| max_{j in S(f(i))} ||k_j - mu||,
    the maximum taken over the row's own slice ("Unchaining the Softmax" ¶3).
    A head is eligible for the fixed max when the largest of its row bounds
    is at most ``beta`` ("Unchaining the Softmax" ¶3: loose heads fall back).

    ``centre=False`` computes the same statistics on the raw keys.
    Returns mu [B,H,d], qnorm [B,H,N], R [B,H,F] (max centred key norm per
    frame), R_S [B,H,F] (max over the slice of frame f), bound [B,H,N],
    stat [B,H] and elig [B,H] (bool), and the same check per (head, frame):
    stat_frame [B,H,F] (the largest row bound among the frame's rows) and
    elig_frame [B,H,F] (bool). A frame passes when each of its rows does, so
    the finer check carries the same guarantee row by row.
    """
    Q = _f64(Q)
    K = _f64(K)
    B, H, N, d = K.shape
    assert N == F * T
    mu = K.mean(axis=-2) if centre else np.zeros((B, H, d))
    R = np.empty((B, H, F))
    for b in range(B):
        for h in range(H):
            kc = K[b, h] - mu[b, h]
            kn = np.sqrt(np.einsum("nd,nd->n", kc, kc))
            R[b, h] = kn.reshape(F, T).max(axis=1)
    R_S = np.empty((B, H, F))
    for f in range(F):
        R_S[:, :, f] = R[:, :, slice_frames(F, window, ref_frame, f)].max(axis=-1)
    qnorm = np.sqrt(np.einsum("bhnd,bhnd->bhn", Q, Q))
    frame_of_row = np.arange(N) // T
    bound = scale * qnorm * R_S[:, :, frame_of_row]
    stat = bound.max(axis=-1)
    stat_frame = bound.reshape(B, H, F, T).max(axis=-1)
    return {"mu": mu, "qnorm": qnorm, "R": R, "R_S": R_S, "bound": bound,
            "stat": stat, "elig": stat <= beta,
            "stat_frame": stat_frame, "elig_frame": stat_frame <= beta}


def gap_bounds(Q, K, F: int, T: int, window: int, ref_frame: int, scale: float,
               limit: float = GAP_LIMIT) -> dict:
    """Per-row bound on how far the fixed max lies above the row's true max.

    In the centred frame ("Unchaining the Softmax" ¶2) the fixed max of row i
    is its Cauchy-Schwarz bound B_i, and the row's largest logit is at least
    the mean of its logits over the slice ("Unchaining the Softmax" ¶3: each
    row sees its own slice), scale <q_i, kbar_S - mu> with kbar_S the mean
    key of the slice S(f(i)). So
        B_i - max_j scale <q_i, k_j - mu>  <=  G_i = B_i - scale <q_i, kbar_S - mu>,
    and 0 <= G_i <= 2 B_i. A row whose G_i is at most ``limit`` may take the
    fixed max with the guarantee the per-head check gives (its largest term
    is at least exp(-limit)).

    Returns dslice [B,H,F,d] (kbar_S(f) - mu), bound [B,H,N] (B_i), gap
    [B,H,N] (G_i) and ok [B,H,N] (G_i <= limit).
    """
    Q = _f64(Q)
    K = _f64(K)
    B, H, N, d = K.shape
    assert N == F * T
    cs = bounds(Q, K, F, T, window, ref_frame, scale)
    mu = cs["mu"]
    frame_mean = K.reshape(B, H, F, T, d).mean(axis=3)          # [B,H,F,d]
    dslice = np.empty((B, H, F, d))
    for f in range(F):
        dslice[:, :, f] = frame_mean[:, :, slice_frames(F, window, ref_frame, f)].mean(axis=2) - mu
    frame_of_row = np.arange(N) // T
    lower = scale * np.einsum("bhnd,bhnd->bhn", Q, dslice[:, :, frame_of_row])
    gap = cs["bound"] - lower
    return {"dslice": dslice, "bound": cs["bound"], "gap": gap, "ok": gap <= limit}


# --------------------------------------------------------------------------
# attention: the definition  ("Deleting the Mask" ¶1)
# --------------------------------------------------------------------------

def _softmax_rows(q, k, v, scale):
    """Exact-max softmax attention of rows q over keys k, values v (fp64)."""
    s = scale * (q @ k.T)
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ v) / p.sum(axis=1, keepdims=True)


def attention_rows(Q, K, V, F: int, T: int, window: int, ref_frame: int,
                   scale: float, b: int, h: int, rows) -> np.ndarray:
    """Output rows ``rows`` of head (b, h): [len(rows), d] in float64."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, K.shape[-1]))
    frames = rows // T
    for f in np.unique(frames):
        sel = np.nonzero(frames == f)[0]
        keys = slice_keys(F, T, window, ref_frame, int(f))
        k = _f64(K[b, h][keys])
        v = _f64(V[b, h][keys])
        for c in range(0, sel.size, ROW_CHUNK):
            part = sel[c:c + ROW_CHUNK]
            out[part] = _softmax_rows(_f64(Q[b, h][rows[part]]), k, v, scale)
    return out


def attention(Q, K, V, F: int, T: int, window: int, ref_frame: int,
              scale: float) -> np.ndarray:
    """Full output O [B, H, N, d] in float64."""
    B, H, N, d = K.shape
    O = np.empty((B, H, N, d))
    for b in range(B):
        for h in range(H):
            O[b, h] = attention_rows(Q, K, V, F, T, window, ref_frame, scale,
                                     b, h, np.arange(N))
    return O


# --------------------------------------------------------------------------
# the two routes the kernel takes, written plainly  ("Unchaining the Softmax")
# --------------------------------------------------------------------------

def attention_fixed_max(Q, K, V, F, T, window, ref_frame, scale, b, h, rows,
                        bnd=None) -> np.ndarray:
    """Fixed-max route: centred keys and a per-row max fixed in advance.

    Each row uses its Cauchy-Schwarz bound as the softmax shift, so no running
    max is kept ("Unchaining the Softmax" ¶2). Equal to the definition in
    exact arithmetic.
    """
    if bnd is None:
        bnd = bounds(Q[b:b + 1, h:h + 1], K[b:b + 1, h:h + 1], F, T, window,
                     ref_frame, scale)
    mu = bnd["mu"][0, 0]
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, K.shape[-1]))
    for n, i in enumerate(rows):
        keys = slice_keys(F, T, window, ref_frame, int(i // T))
        kc = _f64(K[b, h][keys]) - mu
        s = scale * (kc @ _f64(Q[b, h][i]))
        p = np.exp(s - bnd["bound"][0, 0, i])
        out[n] = (p @ _f64(V[b, h][keys])) / p.sum()
    return out


def attention_online(Q, K, V, F, T, window, ref_frame, scale, b, h, rows,
                     block: int = 16, centre: bool = True) -> np.ndarray:
    """Online-softmax route: running max, rescaled when a key block raises it.

    Keys of the slice are visited in ascending order, ``block`` at a time; the
    accumulator and the running sum are rescaled whenever the running max
    grows ("Unchaining the Softmax" ¶1).
    """
    Kf = _f64(K[b, h])
    mu = Kf.mean(axis=0) if centre else np.zeros(Kf.shape[1])
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, Kf.shape[1]))
    for n, i in enumerate(rows):
        keys = slice_keys(F, T, window, ref_frame, int(i // T))
        q = _f64(Q[b, h][i])
        m = -np.inf
        l = 0.0
        acc = np.zeros(Kf.shape[1])
        for c in range(0, keys.size, block):
            kk = keys[c:c + block]
            s = scale * ((Kf[kk] - mu) @ q)
            m_new = max(m, s.max())
            alpha = np.exp(m - m_new)
            p = np.exp(s - m_new)
            l = l * alpha + p.sum()
            acc = acc * alpha + p @ _f64(V[b, h][kk])
            m = m_new
        out[n] = acc / l
    return out


def attention_two_pass(Q, K, V, F, T, window, ref_frame, scale, b, h, rows,
                       add_ref_always: bool = False) -> np.ndarray:
    """The older route: window pass and reference pass merged by log-sum-exp.

    This is the two-pass scheme that frame alignment replaces ("Deleting the
    Mask" ¶1); it serves as a cross-check. The reference pass is skipped when
    the reference frame already lies in the window, unless
    ``add_ref_always`` (which double-counts those keys).
    """
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, K.shape[-1]))
    for n, i in enumerate(rows):
        f = int(i // T)
        lo, hi = max(0, f - window), min(F - 1, f + window)
        q = _f64(Q[b, h][i])
        parts = [np.arange(lo * T, (hi + 1) * T)]
        if add_ref_always or not (lo <= ref_frame <= hi):
            parts.append(np.arange(ref_frame * T, (ref_frame + 1) * T))
        lses, outs = [], []
        for keys in parts:
            s = scale * (_f64(K[b, h][keys]) @ q)
            m = s.max()
            p = np.exp(s - m)
            lses.append(m + np.log(p.sum()))
            outs.append((p @ _f64(V[b, h][keys])) / p.sum())
        lse = np.logaddexp.reduce(lses)
        out[n] = sum(np.exp(l_ - lse) * o for l_, o in zip(lses, outs))
    return out


# --------------------------------------------------------------------------
# cross-attention to a reference token set: another attention variant of the
# pipeline ("The Workload, and the Port" ¶1-¶2: each attention variant gets a
# kernel built for its shape; the product conditions on one photo)
# --------------------------------------------------------------------------

def cross_attention_rows(Q, Kr, Vr, scale: float, b: int, h: int, rows) -> np.ndarray:
    """Rows ``rows`` of O[b, h] for cross-attention: every query row attends
    to all M reference tokens, O_i = softmax_j(scale <q_i, kr_j>) vr. Float64."""
    rows = np.asarray(rows, dtype=np.int64)
    k = _f64(Kr[b, h])
    v = _f64(Vr[b, h])
    out = np.empty((rows.size, k.shape[1]))
    for c in range(0, rows.size, ROW_CHUNK):
        part = rows[c:c + ROW_CHUNK]
        out[c:c + ROW_CHUNK] = _softmax_rows(_f64(Q[b, h][part]), k, v, scale)
    return out


def cross_attention(Q, Kr, Vr, scale: float) -> np.ndarray:
    """Full cross-attention output [B, H, N, d] in float64."""
    B, H, N, d = Q.shape
    O = np.empty((B, H, N, d))
    for b in range(B):
        for h in range(H):
            O[b, h] = cross_attention_rows(Q, Kr, Vr, scale, b, h, np.arange(N))
    return O


def cross_plan(F: int, T: int, M: int, bq: int, bk: int) -> dict:
    """Tile list of cross-attention in the same CSR form as ``plan``: q-blocks
    of bq chunk tokens against k-blocks of bk reference tokens. Every query
    row attends to every reference key, so a tile is live iff it holds a
    valid pair, which every tile does; runs are the one range [0, M)."""
    if bq % 16 or bk % 16 or T % bq or M % bk:
        raise ValueError("bq: multiple of 16 dividing T; bk: multiple of 16 dividing M")
    nqb, nkb = F * T // bq, M // bk
    mask = np.ones((F * T, M), dtype=bool)        # the definition: every pair attends
    row_ptr, col_idx, runs = [0], [], []
    for qb in range(nqb):
        cols = [kb for kb in range(nkb)
                if mask[qb * bq:(qb + 1) * bq, kb * bk:(kb + 1) * bk].any()]
        col_idx.extend(cols)
        row_ptr.append(len(col_idx))
        runs.append([(cols[0] * bk, (cols[-1] + 1) * bk)])
    return {
        "row_ptr": np.asarray(row_ptr, dtype=np.int64),
        "col_idx": np.asarray(col_idx, dtype=np.int64),
        "qframe": np.arange(nqb, dtype=np.int64) * bq // T,
        "runs": runs,
        "nnz": len(col_idx),
    }


def cross_bounds(Q, Kr, F: int, T: int, scale: float, beta: float = BETA) -> dict:
    """Cauchy-Schwarz bounds of cross-attention. The reference keys are
    centred on their own mean mu (softmax-invariant: the row's logits all move
    by scale <q_i, mu>); every row sees every reference key, so its bound is
    scale ||q_i|| R with R = max_j ||kr_j - mu|| ("Unchaining the Softmax"
    ¶2-¶3). Eligibility per head (stat = max_i bound_i <= beta) and per query
    frame (stat_frame over the frame's rows), as for self-attention.
    Every row's slice is the whole reference set, whose mean is mu, so the
    row's gap bound (see gap_bounds) is its bound itself.
    Returns mu [B,H,d], qnorm [B,H,N], R [B,H], bound [B,H,N], stat, elig,
    stat_frame [B,H,F], elig_frame, gap [B,H,N] (= bound)."""
    Q = _f64(Q)
    Kr = _f64(Kr)
    B, H, N, d = Q.shape
    assert N == F * T
    mu = Kr.mean(axis=-2)
    kc = Kr - mu[:, :, None, :]
    R = np.sqrt(np.einsum("bhmd,bhmd->bhm", kc, kc)).max(axis=-1)
    qnorm = np.sqrt(np.einsum("bhnd,bhnd->bhn", Q, Q))
    bound = scale * qnorm * R[:, :, None]
    stat = bound.max(axis=-1)
    stat_frame = bound.reshape(B, H, F, T).max(axis=-1)
    return {"mu": mu, "qnorm": qnorm, "R": R, "bound": bound, "stat": stat,
            "elig": stat <= beta, "stat_frame": stat_frame,
            "elig_frame": stat_frame <= beta, "gap": bound.copy()}
