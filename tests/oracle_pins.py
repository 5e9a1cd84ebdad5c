"""Pins for the fp64 oracle: facts about exact attention that do not come from it.

Each ``pin_*`` takes an oracle object (the ``oracle`` module or an
``oracle.Oracle`` bound to a modified build) and raises AssertionError when
the oracle disagrees with the fact.  tests/test_oracle.py runs them on the
oracle; tests/test_oracle_mutants.py plants mistakes in copies of the oracle
and checks that some pin fails for each.

Sources of truth used here:
  * brute force with a *different* softmax formula: exp(s_j) / fsum(exp(s)),
    no max subtraction, pure Python scalars (the plain softmax of
    "FlashAttention: ... IO-Awareness" section 1.1 instead of the stable form
    of its section 2.4 that the oracle uses);
  * closed forms and invariances of softmax attention;
  * the running-max/running-sum loop of "FlashAttention 深度解析" section 二
    must reach the one-shot result (that page and the IO-Awareness page
    section 2.4 state that the chunked result is identical);
  * central finite differences of L = sum(dO * O) for the backward.
"""
from __future__ import annotations

import math

import numpy as np

MB = 128  # block-mask granularity


def _rng(seed):
    return np.random.default_rng(seed)


def _allowed(i, j, causal, mask, window=None):
    if causal and j > i:
        return False
    if mask is not None and not mask[i // MB, j // MB]:
        return False
    if window is not None:
        # local window: keys from i - left to i + right (None or < 0: unbounded)
        left, right = window
        if left is not None and left >= 0 and j < i - left:
            return False
        if right is not None and right >= 0 and j > i + right:
            return False
    return True


def brute_force_head(q, k, v, scale, causal=False, mask=None, window=None, slope=0.0):
    """Pure-Python scalar attention for one head with exp(s)/fsum(exp(s)).

    ``slope``: ALiBi, the score of (i, j) gets -slope * |i - j| after scaling.
    """
    N, d = q.shape
    o = [[0.0] * d for _ in range(N)]
    lse = [0.0] * N
    for i in range(N):
        cols = [j for j in range(N) if _allowed(i, j, causal, mask, window)]
        if not cols:
            lse[i] = -math.inf
            continue
        e = []
        for j in cols:
            s = scale * math.fsum(float(q[i, c]) * float(k[j, c]) for c in range(d)) - slope * abs(i - j)
            e.append(math.exp(s))
        z = math.fsum(e)
        for c in range(d):
            o[i][c] = math.fsum(e[t] / z * float(v[cols[t], c]) for t in range(len(cols)))
        lse[i] = math.log(z)
    return np.array(o), np.array(lse)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), f"{what}: non-finite pattern differs"
    assert np.array_equal(a[~fin], b[~fin]), f"{what}: infinities differ"
    if fin.any():
        err = np.max(np.abs(a[fin] - b[fin]) / np.maximum(1.0, np.abs(b[fin])))
        assert err <= tol, f"{what}: rel err {err:.3e} > {tol:.1e}"


# ----------------------------------------------------------------------------
# Forward
# ----------------------------------------------------------------------------

def pin_brute_force(orc):
    """Tiny dense/causal cases and >128-row block-mask cases vs the brute force."""
    cases = []
    for seed, (N, d, scale, causal) in enumerate(
            [(1, 1, 1.0, False), (5, 3, 0.5, False), (8, 4, 1.0, True), (7, 2, 0.5, True),
             (8, 4, 0.5, False)]):
        cases.append((N, d, scale, causal, None, seed))
    # block masks need N > 128 to have more than one block
    r = _rng(99)
    for seed, (N, causal) in enumerate([(200, False), (260, True), (257, False)]):
        nb = (N + MB - 1) // MB
        mask = (r.random((nb, nb)) < 0.6).astype(np.uint8)
        mask[0, 0] = 1
        cases.append((N, 2, 0.7, causal, mask, 100 + seed))
    # a row with no allowed key at all
    mask = np.array([[1, 0], [0, 0]], dtype=np.uint8)
    cases.append((150, 2, 1.0, False, mask, 200))
    for N, d, scale, causal, mask, seed in cases:
        g = _rng(seed)
        q, k, v = (g.standard_normal((1, 1, N, d)) for _ in range(3))
        o, lse = orc.attn_fwd(q, k, v, scale, causal, mask)
        ob, lb = brute_force_head(q[0, 0], k[0, 0], v[0, 0], scale, causal, mask)
        _close(o[0, 0], ob, 1e-12, f"O N={N} d={d} causal={causal} mask={mask is not None}")
        _close(lse[0, 0], lb, 1e-12, f"lse N={N}")


def pin_rows_sum_to_one(orc):
    """Rows of P are a probability distribution over exactly the allowed keys."""
    g = _rng(1)
    N, d = 300, 8
    q, k = g.standard_normal((N, d)), g.standard_normal((N, d))
    nb = 3
    mask = (g.random((nb, nb)) < 0.7).astype(np.uint8)
    np.fill_diagonal(mask, 1)
    for causal in (False, True):
        for m in (None, mask):
            P, lse = orc.attn_probs(q, k, 0.35, causal, m)
            allowed = np.array([[_allowed(i, j, causal, m) for j in range(N)] for i in range(N)])
            assert np.all(P[~allowed] == 0.0)
            assert np.all(P[allowed] > 0.0)
            assert np.max(np.abs(P.sum(axis=1) - 1.0)) <= 1e-12


def pin_constant_v(orc):
    """V_j = c for every key makes every output row equal c (convex combination)."""
    g = _rng(2)
    B, H, N, d = 2, 2, 96, 16
    q, k = g.standard_normal((B, H, N, d)), g.standard_normal((B, H, N, d))
    c = g.standard_normal(d)
    v = np.broadcast_to(c, (B, H, N, d)).copy()
    for causal in (False, True):
        o, _ = orc.attn_fwd(q, k, v, 0.25, causal)
        assert np.max(np.abs(o - c)) <= 1e-12


def pin_causal_first_row(orc):
    """With a causal mask row 0 sees only key 0: O_0 = V_0 and lse_0 = s q_0.k_0."""
    g = _rng(3)
    B, H, N, d = 1, 3, 64, 32
    q, k, v = (g.standard_normal((B, H, N, d)) for _ in range(3))
    s = 0.125
    o, lse = orc.attn_fwd(q, k, v, s, causal=True)
    assert np.max(np.abs(o[:, :, 0] - v[:, :, 0])) <= 1e-12
    want = s * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0])
    assert np.max(np.abs(lse[:, :, 0] - want)) <= 1e-12


def pin_chunked_equals_one_shot(orc):
    """The online loop with any chunk size reaches the one-shot result."""
    g = _rng(4)
    B, H, N, d = 1, 2, 300, 16
    q, k, v = (g.standard_normal((B, H, N, d)) * 1.5 for _ in range(3))
    nb = 3
    mask = (g.random((nb, nb)) < 0.7).astype(np.uint8)
    np.fill_diagonal(mask, 1)
    for causal, m in ((False, None), (True, None), (False, mask), (True, mask)):
        o, lse = orc.attn_fwd(q, k, v, 0.3, causal, m)
        for chunk in (1, 7, 64, 128, N):
            o2, l2 = orc.attn_fwd_online(q, k, v, 0.3, chunk, causal, m)
            _close(o2, o, 1e-12, f"online chunk={chunk}")
            _close(l2, lse, 1e-12, f"online lse chunk={chunk}")


def pin_closed_forms(orc):
    g = _rng(5)
    # N = 1: O = V_0, lse = s q.k
    q, k, v = (g.standard_normal((2, 1, 1, 8)) for _ in range(3))
    o, lse = orc.attn_fwd(q, k, v, 0.7)
    assert np.max(np.abs(o - v)) <= 1e-15
    assert np.max(np.abs(lse - 0.7 * np.einsum("bhnd,bhnd->bhn", q, k))) <= 1e-12
    # scale = 0: uniform weights over the allowed set
    B, H, N, d = 1, 1, 200, 4
    q, k, v = (g.standard_normal((B, H, N, d)) for _ in range(3))
    mask = np.array([[1, 0], [1, 1]], dtype=np.uint8)
    for causal, m in ((False, None), (True, None), (False, mask), (True, mask)):
        o, lse = orc.attn_fwd(q, k, v, 0.0, causal, m)
        for i in range(N):
            cols = [j for j in range(N) if _allowed(i, j, causal, m)]
            assert abs(lse[0, 0, i] - math.log(len(cols))) <= 1e-12
            want = v[0, 0, cols].mean(axis=0)
            assert np.max(np.abs(o[0, 0, i] - want)) <= 1e-12
    # one-hot: one score exceeds every other by more than 60 -> O_i = V_j*.
    # Key j carries a unit marker in coordinate j; query i puts 100 on the marker
    # of its chosen key star[i]; the remaining coordinates are small noise.
    N = 32
    star = g.integers(0, N, size=N)
    noise = 0.1 * g.standard_normal((1, 1, N, 4))
    q = np.concatenate([noise, np.zeros((1, 1, N, N))], axis=3)
    k = np.concatenate([0.1 * g.standard_normal((1, 1, N, 4)), np.eye(N)[None, None]], axis=3)
    v = g.standard_normal((1, 1, N, 4 + N))
    for i in range(N):
        q[0, 0, i, 4 + star[i]] = 100.0
    o, _ = orc.attn_fwd(q, k, v, 1.0)
    for i in range(N):
        assert np.max(np.abs(o[0, 0, i] - v[0, 0, star[i]])) <= 1e-12


def pin_invariances(orc):
    g = _rng(6)
    B, H, N, d = 1, 2, 260, 8
    q, k, v = (g.standard_normal((B, H, N, d)) for _ in range(3))
    s = 0.4
    # shifting every key by the same vector shifts each score row by a constant
    shift = g.standard_normal(d)
    for causal in (False, True):
        o, lse = orc.attn_fwd(q, k, v, s, causal)
        o2, lse2 = orc.attn_fwd(q, k + shift, v, s, causal)
        _close(o2, o, 1e-12, "key shift O")
        _close(lse2, lse + s * np.einsum("bhnd,d->bhn", q, shift), 1e-12, "key shift lse")
    # jointly permuting keys and values leaves a non-causal, unmasked output unchanged
    perm = g.permutation(N)
    o, lse = orc.attn_fwd(q, k, v, s)
    o2, lse2 = orc.attn_fwd(q, k[:, :, perm], v[:, :, perm], s)
    _close(o2, o, 1e-12, "perm O")
    _close(lse2, lse, 1e-12, "perm lse")
    # an all-ones block mask is the dense case
    nb = 3
    ones = np.ones((nb, nb), dtype=np.uint8)
    for causal in (False, True):
        o, lse = orc.attn_fwd(q, k, v, s, causal)
        o2, lse2 = orc.attn_fwd(q, k, v, s, causal, ones)
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    # a block mask equals dense attention with an additive -inf bias (numpy route)
    mask = (g.random((nb, nb)) < 0.5).astype(np.uint8)
    mask[:, 0] = 1
    o, lse = orc.attn_fwd(q, k, v, s, False, mask)
    bias = np.where(np.kron(mask, np.ones((MB, MB)))[:N, :N] > 0, 0.0, -np.inf)
    for bh in range(B * H):
        b, h = divmod(bh, H)
        S = s * q[b, h] @ k[b, h].T + bias
        mx = S.max(axis=1, keepdims=True)
        E = np.exp(S - mx)
        Z = E.sum(axis=1, keepdims=True)
        _close(o[b, h], (E / Z) @ v[b, h], 1e-12, "additive mask O")
        _close(lse[b, h], (mx + np.log(Z))[:, 0], 1e-12, "additive mask lse")


def pin_rows_match_full(orc):
    """The sampled-row entry point agrees with the full forward on those rows."""
    g = _rng(7)
    B, H, N, d = 2, 2, 270, 8
    q, k, v = (g.standard_normal((B, H, N, d)) for _ in range(3))
    nb = 3
    mask = (g.random((nb, nb)) < 0.6).astype(np.uint8)
    mask[2, :] = 0  # rows of the last block see nothing
    rows = np.array([[0, 0], [1, 5], [3, 269], [2, 128], [3, 127], [0, 256]], dtype=np.int64)
    for causal, m in ((False, None), (True, None), (True, mask)):
        o, lse = orc.attn_fwd(q, k, v, 0.3, causal, m)
        orow, lrow = orc.attn_fwd_rows(q, k, v, 0.3, rows, causal, m)
        of = o.reshape(B * H, N, d)
        lf = lse.reshape(B * H, N)
        for r, (bh, i) in enumerate(rows):
            assert np.array_equal(orow[r], of[bh, i])
            assert lrow[r] == lf[bh, i] or (np.isinf(lrow[r]) and np.isinf(lf[bh, i]))


# ----------------------------------------------------------------------------
# Backward
# ----------------------------------------------------------------------------

def pin_finite_differences(orc):
    """dQ, dK, dV equal central differences of L = sum(dO * O)."""
    g = _rng(8)
    h = 1e-6
    for N, d, causal, m in ((6, 3, False, None), (9, 4, True, None), (16, 8, True, None),
                            (140, 2, False, np.array([[1, 0], [1, 1]], dtype=np.uint8))):
        q, k, v, do = (g.standard_normal((1, 1, N, d)) for _ in range(4))
        s = 0.6
        dq, dk, dv = orc.attn_bwd(q, k, v, do, s, causal, m)

        def loss(qq, kk, vv):
            o, _ = orc.attn_fwd(qq, kk, vv, s, causal, m)
            return float(np.sum(do * o))

        # every coordinate on the tiny cases, a seeded subset on the bigger one
        coords = [(i, c) for i in range(N) for c in range(d)]
        if N > 32:
            pick = g.choice(len(coords), size=24, replace=False)
            coords = [coords[t] for t in pick]
        for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            for i, c in coords:
                xp, xm = x.copy(), x.copy()
                xp[0, 0, i, c] += h
                xm[0, 0, i, c] -= h
                args_p = {"q": q, "k": k, "v": v}
                args_m = {"q": q, "k": k, "v": v}
                args_p[name], args_m[name] = xp, xm
                fd = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                      loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
                an = grad[0, 0, i, c]
                assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, N, i, c, fd, an)


def pin_backward_identities(orc):
    g = _rng(9)
    B, H, N, d = 1, 2, 200, 8
    q, k, v, do = (g.standard_normal((B, H, N, d)) for _ in range(4))
    nb = 2
    mask = np.array([[1, 1], [0, 1]], dtype=np.uint8)
    for causal, m in ((False, None), (True, None), (True, mask)):
        dq, dk, dv, o, lse, D = orc.attn_bwd(q, k, v, do, 0.3, causal, m, return_fwd=True)
        o_f, lse_f = orc.attn_fwd(q, k, v, 0.3, causal, m)
        assert np.max(np.abs(o - o_f)) <= 1e-14 and np.max(np.abs(lse - lse_f)) <= 1e-14
        # D_i = sum_j P_ij dP_ij equals rowsum(dO * O)
        _close(D, np.sum(do * o, axis=-1), 1e-10, "D = rowsum(dO*O)")
        # sum_j dK_j = 0 (softmax rows are shift invariant)
        assert np.max(np.abs(dk.sum(axis=2))) <= 1e-10
        # sum_j dV_j = sum_i dO_i (rows of P sum to 1)
        assert np.max(np.abs(dv.sum(axis=2) - do.sum(axis=2))) <= 1e-10


# ----------------------------------------------------------------------------
# Local window and ALiBi (the further built-in variants of "FlashAttention
# 深度解析" section 五)
# ----------------------------------------------------------------------------

def pin_window_alibi_brute_force(orc):
    """Window and ALiBi (alone and combined, with causal and a block mask) vs the brute force."""
    g = _rng(21)
    cases = [(9, 3, False, None, (2, 1), None), (9, 3, True, None, (3, -1), None),
             (9, 3, False, None, None, (0.3, 1.1)), (12, 4, True, None, (4, -1), (0.7, 0.05)),
             (10, 2, False, None, (0, 0), (0.5, 0.5)), (11, 3, False, None, (-1, 2), (1.5, 0.0)),
             (140, 2, False, np.array([[1, 0], [1, 1]], dtype=np.uint8), (60, 5), (0.02, 0.2))]
    for N, d, causal, m, window, slopes in cases:
        q, k, v = (g.standard_normal((1, 2, N, d)) for _ in range(3))
        o, lse = orc.attn_fwd(q, k, v, 0.7, causal, m, window=window, slopes=slopes)
        for h in range(2):
            sl = 0.0 if slopes is None else slopes[h]
            ob, lb = brute_force_head(q[0, h], k[0, h], v[0, h], 0.7, causal, m, window, sl)
            _close(o[0, h], ob, 1e-12, f"window/alibi O N={N} h={h}")
            _close(lse[0, h], lb, 1e-12, f"window/alibi lse N={N} h={h}")


def pin_window_special_cases(orc):
    """Window (inf, 0) = causal; a window wider than N = no window; window (0, 0)
    keeps only the diagonal: O_i = V_i and lse_i = scale q_i.k_i (ALiBi adds 0 there)."""
    g = _rng(22)
    N, d = 37, 5
    q, k, v = (g.standard_normal((1, 2, N, d)) for _ in range(3))
    o_c, l_c = orc.attn_fwd(q, k, v, 0.4, True)
    o_w, l_w = orc.attn_fwd(q, k, v, 0.4, False, window=(-1, 0))
    _close(o_w, o_c, 1e-15, "window (inf, 0) = causal")
    _close(l_w, l_c, 1e-15, "window (inf, 0) = causal lse")
    o_d, l_d = orc.attn_fwd(q, k, v, 0.4, False)
    o_n, l_n = orc.attn_fwd(q, k, v, 0.4, False, window=(N, N + 3))
    _close(o_n, o_d, 1e-15, "wide window = dense")
    _close(l_n, l_d, 1e-15, "wide window = dense lse")
    o_0, l_0 = orc.attn_fwd(q, k, v, 0.4, False, window=(0, 0), slopes=(0.9, 2.0))
    _close(o_0, v, 1e-14, "window (0, 0): O = V")
    _close(l_0, 0.4 * np.einsum("bhnd,bhnd->bhn", q, k), 1e-13, "window (0, 0): lse = s q.k")


def pin_alibi_closed_form(orc):
    """Scale 0 leaves only the bias: with two keys P_i = softmax(0, -m) in key order
    of distance, O and lse in closed form; slope 0 equals no ALiBi."""
    g = _rng(23)
    d = 4
    q, k, v = (g.standard_normal((1, 1, 2, d)) for _ in range(3))
    m = 0.8
    o, lse = orc.attn_fwd(q, k, v, 0.0, False, slopes=(m,))
    e = math.exp(-m)
    _close(o[0, 0, 0], (v[0, 0, 0] + e * v[0, 0, 1]) / (1 + e), 1e-14, "alibi row 0")
    _close(o[0, 0, 1], (e * v[0, 0, 0] + v[0, 0, 1]) / (1 + e), 1e-14, "alibi row 1")
    _close(lse[0, 0], [math.log1p(e)] * 2, 1e-14, "alibi lse")
    q, k, v = (g.standard_normal((1, 3, 30, d)) for _ in range(3))
    o1, l1 = orc.attn_fwd(q, k, v, 0.5, True, slopes=(0.0, 0.0, 0.0))
    o2, l2 = orc.attn_fwd(q, k, v, 0.5, True)
    _close(o1, o2, 1e-15, "slope 0 = no alibi")
    _close(l1, l2, 1e-15, "slope 0 = no alibi lse")


def pin_alibi_is_additive_bias(orc):
    """ALiBi is exactly the additive bias -m_h |i - j|: a numpy softmax of the
    biased, window-masked score matrix gives the same O and lse."""
    g = _rng(24)
    B, H, N, d = 1, 3, 150, 6
    q, k, v = (g.standard_normal((B, H, N, d)) for _ in range(3))
    slopes = np.array([0.01, 0.25, 1.0])
    window = (40, 7)
    o, lse = orc.attn_fwd(q, k, v, 0.35, False, window=window, slopes=slopes)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    keep = (j >= i - window[0]) & (j <= i + window[1])
    for h in range(H):
        s = 0.35 * (q[0, h] @ k[0, h].T) - slopes[h] * np.abs(i - j)
        s = np.where(keep, s, -np.inf)
        mx = s.max(axis=1, keepdims=True)
        e = np.exp(s - mx)
        z = e.sum(axis=1, keepdims=True)
        _close(o[0, h], (e / z) @ v[0, h], 1e-12, f"alibi bias O h={h}")
        _close(lse[0, h], (mx + np.log(z))[:, 0], 1e-12, f"alibi bias lse h={h}")


def pin_window_alibi_chunked_and_rows(orc):
    """The online loop and the sampled-row entry point agree with the one-shot
    forward under window + ALiBi."""
    g = _rng(25)
    B, H, N, d = 1, 2, 300, 4
    q, k, v = (g.standard_normal((B, H, N, d)) for _ in range(3))
    kw = dict(window=(70, 3), slopes=(0.05, 0.3))
    o, lse = orc.attn_fwd(q, k, v, 0.5, True, **kw)
    for chunk in (1, 13, 128):
        oc, lc = orc.attn_fwd_online(q, k, v, 0.5, chunk, True, **kw)
        _close(oc, o, 1e-12, f"online chunk={chunk}")
        _close(lc, lse, 1e-12, f"online lse chunk={chunk}")
    rows = np.array([[0, 0], [1, 5], [0, 150], [1, 299], [1, 71]], dtype=np.int64)
    orr, lrr = orc.attn_fwd_rows(q, k, v, 0.5, rows, True, **kw)
    for t, (bh, i) in enumerate(rows):
        _close(orr[t], o[0, bh, i], 1e-14, "rows O")
        _close(lrr[t], lse[0, bh, i], 1e-14, "rows lse")


def pin_window_alibi_finite_differences(orc):
    """dQ, dK, dV under window + ALiBi equal central differences of sum(dO * O)."""
    g = _rng(26)
    h = 1e-6
    for N, d, causal, window, slopes in ((8, 3, False, (2, 1), (0.4,)), (11, 2, True, (3, -1), (1.2,))):
        q, k, v, do = (g.standard_normal((1, 1, N, d)) for _ in range(4))
        s = 0.6
        kw = dict(window=window, slopes=slopes)
        dq, dk, dv = orc.attn_bwd(q, k, v, do, s, causal, None, **kw)

        def loss(qq, kk, vv):
            o, _ = orc.attn_fwd(qq, kk, vv, s, causal, None, **kw)
            return float(np.sum(do * o))

        for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            for i in range(N):
                for c in range(d):
                    xp, xm = x.copy(), x.copy()
                    xp[0, 0, i, c] += h
                    xm[0, 0, i, c] -= h
                    a_p = {"q": q, "k": k, "v": v}
                    a_m = {"q": q, "k": k, "v": v}
                    a_p[name], a_m[name] = xp, xm
                    fd = (loss(a_p["q"], a_p["k"], a_p["v"]) - loss(a_m["q"], a_m["k"], a_m["v"])) / (2 * h)
                    an = grad[0, 0, i, c]
                    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, N, i, c, fd, an)


# ---------------------------------------------------------------------------
# Decode over a paged KV cache ("FlashAttention 深度解析" section 五: the
# paged KV-cache interface).  Sources of truth: brute force that assembles each
# sequence's keys page by page in Python with the plain softmax formula; the
# square oracle (already pinned above) on contiguous pages; invariances.
# ---------------------------------------------------------------------------

def _paged_case(seed, B, H, Hkv, Nq, d, page_size, num_pages, max_pages, lens):
    r = _rng(seed)
    q = r.standard_normal((B, H, Nq, d))
    kc = r.standard_normal((num_pages, page_size, Hkv, d))
    vc = r.standard_normal((num_pages, page_size, Hkv, d))
    # distinct physical pages per sequence, in a shuffled order
    perm = r.permutation(num_pages)
    bt = np.full((B, max_pages), -7, dtype=np.int32)  # unused entries hold garbage
    used = 0
    for b in range(B):
        need = -(-lens[b] // page_size)
        bt[b, :need] = perm[used:used + need]
        used += need
    return q, kc, vc, bt, np.array(lens, dtype=np.int32)


def _paged_brute(q, kc, vc, bt, lens, scale, causal):
    B, H, Nq, d = q.shape
    page_size, Hkv = kc.shape[1], kc.shape[2]
    G = H // Hkv
    o = np.zeros_like(q)
    lse = np.zeros((B, H, Nq))
    for b in range(B):
        L = int(lens[b])
        keys, vals = [], []
        for t in range(L):
            page = int(bt[b, t // page_size])
            keys.append(kc[page, t % page_size])
            vals.append(vc[page, t % page_size])
        for h in range(H):
            for i in range(Nq):
                last = L - Nq + i if causal else L - 1
                cols = list(range(0, min(last, L - 1) + 1))
                if not cols:
                    lse[b, h, i] = -math.inf
                    continue
                e = [math.exp(scale * math.fsum(float(q[b, h, i, c]) * float(keys[t][h // G, c]) for c in range(d)))
                     for t in cols]
                z = math.fsum(e)
                for c in range(d):
                    o[b, h, i, c] = math.fsum(e[u] / z * float(vals[t][h // G, c]) for u, t in enumerate(cols))
                lse[b, h, i] = math.log(z)
    return o, lse


def pin_paged_brute_force(orc):
    """Grouped heads, several page sizes, lengths that end inside a page, a
    length shorter than the query count (first queries see nothing), an
    empty sequence; causal and not."""
    cases = [
        # B, H, Hkv, Nq, d, page_size, num_pages, max_pages, lens
        (3, 4, 2, 3, 8, 4, 12, 4, [13, 2, 0]),
        (2, 3, 3, 1, 5, 8, 6, 3, [17, 24]),
        (2, 6, 1, 2, 4, 2, 20, 10, [7, 19]),
    ]
    for seed, (B, H, Hkv, Nq, d, ps, npg, mp, lens) in enumerate(cases):
        q, kc, vc, bt, sl = _paged_case(100 + seed, B, H, Hkv, Nq, d, ps, npg, mp, lens)
        for causal in (False, True):
            o, lse = orc.attn_paged_fwd(q, kc, vc, bt, sl, 0.6, causal)
            ob, lb = _paged_brute(q, kc, vc, bt, sl, 0.6, causal)
            _close(o, ob, 1e-12, f"paged O case {seed} causal={causal}")
            _close(lse, lb, 1e-12, f"paged lse case {seed} causal={causal}")


def pin_paged_equals_square(orc):
    """Contiguous pages in order, one KV head per query head and every position
    a query: decode is the square causal (and dense) attention."""
    B, H, N, d, ps = 2, 3, 40, 16, 8
    r = _rng(110)
    q = r.standard_normal((B, H, N, d))
    k = r.standard_normal((B, H, N, d))
    v = r.standard_normal((B, H, N, d))
    npg = B * N // ps
    kc = np.zeros((npg, ps, H, d))
    vc = np.zeros((npg, ps, H, d))
    bt = np.zeros((B, N // ps), dtype=np.int32)
    for b in range(B):
        for p in range(N // ps):
            bt[b, p] = b * (N // ps) + p
            kc[bt[b, p]] = k[b, :, p * ps:(p + 1) * ps].transpose(1, 0, 2)
            vc[bt[b, p]] = v[b, :, p * ps:(p + 1) * ps].transpose(1, 0, 2)
    sl = np.full(B, N, dtype=np.int32)
    for causal in (True, False):
        o, lse = orc.attn_paged_fwd(q, kc, vc, bt, sl, 0.45, causal)
        o2, l2 = orc.attn_fwd(q, k, v, 0.45, causal)
        _close(o, o2, 1e-13, f"paged = square causal={causal}")
        _close(lse, l2, 1e-13, f"paged lse = square causal={causal}")


def pin_paged_invariances(orc):
    """Moving pages to other physical slots (table updated) and NaN in every
    cache row no sequence owns change nothing; repeating each KV head G times
    equals grouped heads; a single query sees all keys with or without causal."""
    B, H, Hkv, Nq, d, ps, npg, mp = 2, 4, 2, 2, 8, 4, 16, 6
    q, kc, vc, bt, sl = _paged_case(120, B, H, Hkv, Nq, d, ps, npg, mp, [21, 10])
    o, lse = orc.attn_paged_fwd(q, kc, vc, bt, sl, 0.5, True)
    # relocate: physical page p -> perm[p], cache rows past each length and unused pages -> NaN
    perm = _rng(121).permutation(npg)
    kc2 = np.full_like(kc, np.nan)
    vc2 = np.full_like(vc, np.nan)
    bt2 = bt.copy()
    for b in range(B):
        for pgi in range(-(-int(sl[b]) // ps)):
            src = bt[b, pgi]
            dst = perm[src]
            bt2[b, pgi] = dst
            rows = min(ps, int(sl[b]) - pgi * ps)
            kc2[dst, :rows] = kc[src, :rows]
            vc2[dst, :rows] = vc[src, :rows]
    o2, l2 = orc.attn_paged_fwd(q, kc2, vc2, bt2, sl, 0.5, True)
    _close(o2, o, 0.0, "paged relocation / NaN outside the sequences")
    _close(l2, lse, 0.0, "paged lse relocation")
    # grouped heads = KV heads repeated
    G = H // Hkv
    o3, l3 = orc.attn_paged_fwd(q, np.repeat(kc, G, axis=2), np.repeat(vc, G, axis=2), bt, sl, 0.5, True)
    _close(o3, o, 1e-14, "grouped heads = repeated KV heads")
    _close(l3, lse, 1e-14, "grouped heads lse")
    # one query: causal and dense agree
    o4, l4 = orc.attn_paged_fwd(q[:, :, :1], kc, vc, bt, sl, 0.5, True)
    o5, l5 = orc.attn_paged_fwd(q[:, :, :1], kc, vc, bt, sl, 0.5, False)
    _close(o4, o5, 0.0, "single query causal = dense")
    _close(l4, l5, 0.0, "single query lse")


# ---------------------------------------------------------------------------
# FP8 block quantization and incoherent processing ("FlashAttention 深度解析"
# section 四).  Sources of truth: torch's float8_e4m3fn conversion (an
# independent implementation of the OCP E4M3 format), scipy's Hadamard
# matrix, exactness properties, and the pages' statement that block
# quantization with incoherent processing has lower error than plain FP8.
# ---------------------------------------------------------------------------

def pin_e4m3_format(orc):
    import torch
    codes = np.arange(256, dtype=np.uint8)
    mine = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref)), "NaN codes"
    fin = ~np.isnan(ref)
    assert np.array_equal(mine[fin], ref[fin]), "E4M3 code values"
    assert mine[0x38] == 1.0 and mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6
    # encoding: round to nearest even within range (torch rounds the same way), saturation above
    x = np.concatenate([np.linspace(-448, 448, 20001), _rng(130).standard_normal(5000) * 3,
                        _rng(131).standard_normal(2000) * 1e-3, mine[fin],
                        (mine[fin][:-1] + mine[fin][1:]) / 2])  # exact midpoints of neighbours
    x = x[np.abs(x) <= 448]
    enc = orc.e4m3_encode(x)
    tref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch maps -0.0 results to 0x80 too; compare values, then signs of zeros
    assert np.array_equal(orc.e4m3_decode(enc), torch.from_numpy(tref).view(torch.float8_e4m3fn)
                          .to(torch.float64).numpy()), "E4M3 rounding"
    sat = orc.e4m3_encode(np.array([448.5, 1e6, -500.0, -1e30]))
    assert sat.tolist() == [0x7E, 0x7E, 0xFE, 0xFE], "saturation at 448"


def pin_incoherent_map(orc):
    from scipy.linalg import hadamard as sp_hadamard
    for d in (4, 64, 128):
        r = _rng(140 + d)
        x = r.standard_normal((7, d))
        sigma = r.choice([-1.0, 1.0], size=d)
        H = sp_hadamard(d).astype(np.float64)
        _close(orc.hadamard(x, sigma), (x * sigma) @ H.T, 1e-12, f"H (sigma o x), d={d}")
        _close(orc.hadamard(x, sigma, True), (x * sigma) @ H.T / d, 1e-12, f"inverse side, d={d}")
        # the pair of maps leaves every dot product unchanged
        y = r.standard_normal((5, d))
        _close(orc.hadamard(x, sigma) @ orc.hadamard(y, sigma, True).T, x @ y.T, 1e-11, f"QK^T kept, d={d}")


def pin_block_quantization(orc):
    r = _rng(150)
    B, H, N, d, blk = 1, 2, 150, 16, 64
    x = r.standard_normal((B, H, N, d)) * np.exp(r.standard_normal((B, H, N, 1)))
    x[0, 1, 64:128] = 0.0                      # an all-zero block
    x[0, 0, 5, 3] = 1e4                         # an outlier
    codes, exps = orc.fp8_quantize(x, blk)
    assert exps.shape == (1, 2, 3)
    vals = orc.e4m3_decode(codes)
    for h in range(H):
        for bi in range(3):
            blkx = x[0, h, bi * blk:(bi + 1) * blk]
            e = int(exps[0, h, bi])
            amax = np.abs(blkx).max()
            if amax == 0:
                assert e == 0 and np.all(codes[0, h, bi * blk:(bi + 1) * blk] == 0)
                continue
            assert amax / 2.0 ** e <= 448 < amax / 2.0 ** (e - 1), "smallest power-of-two scale"
            # codes are the nearest E4M3 values of x / 2^e
            assert np.array_equal(codes[0, h, bi * blk:(bi + 1) * blk], orc.e4m3_encode(blkx / 2.0 ** e))
            deq = vals[0, h, bi * blk:(bi + 1) * blk] * 2.0 ** e
            # error within half a step of the format at each magnitude (and below the subnormal step)
            mag = np.maximum(np.abs(blkx) / 2.0 ** e, 2.0 ** -6)
            step = 2.0 ** (np.floor(np.log2(mag)) - 3) * 2.0 ** e
            assert np.all(np.abs(deq - blkx) <= step / 2 * (1 + 1e-12)), "within half a step"
    deq_all = orc.fp8_dequantize(codes, exps, blk)
    assert np.array_equal(deq_all, vals * np.exp2(np.repeat(exps.astype(float), blk, axis=2)[:, :, :N])[..., None])


def pin_fp8_attention(orc):
    # values already on the E4M3 grid with every block's largest magnitude in (224, 448]: no rounding
    r = _rng(160)
    B, H, N, d = 1, 2, 96, 16
    grid = orc.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    def on_grid(seed):
        g = _rng(seed).choice(grid[grid <= 8], size=(B, H, N, d)) * _rng(seed + 1).choice([-1, 1], size=(B, H, N, d))
        g[:, :, ::64, 0] = 256.0  # pin each block's amax into (224, 448]
        return g / 64.0 * 64.0
    q, k, v = on_grid(161), on_grid(163), on_grid(165)
    o8, l8, _ = orc.attn_fp8_fwd(q, k, v, 0.003, True, block=64)
    o, l = orc.attn_fwd(q, k, v, 0.003, True)
    _close(o8, o, 0.0, "fp8 path on exact inputs")
    _close(l8, l, 0.0, "fp8 lse on exact inputs")
    # the pages: block quantization with incoherent processing has lower error
    # than plain (per-tensor) FP8, on inputs with rare large entries
    N, d = 256, 64
    def outliers(seed):
        z = _rng(seed).standard_normal((1, 2, N, d))
        m = _rng(seed + 1).random((1, 2, N, d)) < 0.001
        return z + m * _rng(seed + 2).standard_normal((1, 2, N, d)) * 10.0
    sc = 1 / np.sqrt(d)
    for seed in (170, 200, 300):
        q, k, v = outliers(seed), outliers(seed + 3), outliers(seed + 6)
        o_ex, _ = orc.attn_fwd(q, k, v, sc, False)
        sigma = _rng(seed + 9).choice([-1.0, 1.0], size=d)
        o_plain, _, _ = orc.attn_fp8_fwd(q, k, v, sc, False, block=N)
        o_blk, _, _ = orc.attn_fp8_fwd(q, k, v, sc, False, block=64, sigma=sigma)
        e_plain = np.sqrt(np.mean((o_plain - o_ex) ** 2))
        e_blk = np.sqrt(np.mean((o_blk - o_ex) ** 2))
        assert e_blk < 0.9 * e_plain, f"block + incoherent {e_blk:.3e} vs plain {e_plain:.3e}"


ALL_PINS = [
    pin_brute_force,
    pin_rows_sum_to_one,
    pin_constant_v,
    pin_causal_first_row,
    pin_chunked_equals_one_shot,
    pin_closed_forms,
    pin_invariances,
    pin_rows_match_full,
    pin_finite_differences,
    pin_backward_identities,
    pin_window_alibi_brute_force,
    pin_window_special_cases,
    pin_alibi_closed_form,
    pin_alibi_is_additive_bias,
    pin_window_alibi_chunked_and_rows,
    pin_window_alibi_finite_differences,
    pin_paged_brute_force,
    pin_paged_equals_square,
    pin_paged_invariances,
    pin_e4m3_format,
    pin_incoherent_map,
    pin_block_quantization,
    pin_fp8_attention,
]
