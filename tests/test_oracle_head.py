"""Pins of the oracle's steps either side of the layer stack (embedding gather, final
RMSNorm, LM head, greedy token) to closed forms and brute force."""

import numpy as np
import pytest

import oracle


def test_embed_gathers_rows_and_marks_bad_ids():
    E = np.arange(5 * 3, dtype=np.float64).reshape(5, 3) * 0.5 - 2.0
    tokens = np.array([[4, 0, -1], [2, 5, 4]])
    out = oracle.embed(tokens, E)
    assert out.shape == (2, 3, 3)
    for idx in np.ndindex(tokens.shape):
        t = tokens[idx]
        if 0 <= t < 5:
            assert np.array_equal(out[idx], E[t])
        else:
            assert np.isnan(out[idx]).all()


def test_final_norm_closed_forms():
    eps = 1e-6
    w = np.array([1.0, 2.0, -0.5, 3.0])
    for c in (0.3, -7.0, 1e3):
        row = np.full(4, c)
        # mean of squares is c^2, so every element becomes c / sqrt(c^2 + eps) times its weight
        np.testing.assert_allclose(oracle.final_norm(row, w, eps), c / np.sqrt(c * c + eps) * w, rtol=1e-14)
    x = np.random.default_rng(0).standard_normal((3, 64))
    # eps -> 0: the norm is invariant to a positive row scale and gives unit mean square
    y = oracle.final_norm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-12)
    np.testing.assert_allclose(oracle.final_norm(5.0 * x, np.ones(64), 0.0), y, rtol=1e-12)


def test_lm_head_one_hot_rows_select_columns():
    rng = np.random.default_rng(1)
    W = rng.standard_normal((11, 6))
    xn = np.eye(6)[[2, 0, 5]] * np.array([[1.0], [3.0], [-2.0]])
    logits = oracle.lm_head_logits(xn, W)
    np.testing.assert_allclose(logits, np.stack([W[:, 2], 3.0 * W[:, 0], -2.0 * W[:, 5]]), rtol=1e-15)


def test_lm_head_matches_brute_force():
    rng = np.random.default_rng(2)
    xn, W = rng.standard_normal((4, 7)), rng.standard_normal((9, 7))
    got = oracle.lm_head_logits(xn, W)
    for r in range(4):
        for v in range(9):
            assert got[r, v] == pytest.approx(sum(xn[r, k] * W[v, k] for k in range(7)), rel=1e-12, abs=1e-12)


def test_greedy_token_lowest_index_on_ties():
    logits = np.array([[0.5, 2.0, 2.0, -1.0],
                       [3.0, 3.0, 3.0, 3.0],
                       [-5.0, -4.0, -6.0, -4.5]])
    tok, mx = oracle.greedy_tokens(logits)
    assert tok.tolist() == [1, 0, 1]
    assert mx.tolist() == [2.0, 3.0, -4.0]


def test_greedy_token_brute_force():
    rng = np.random.default_rng(3)
    logits = np.round(rng.standard_normal((50, 13)), 1)      # rounded so ties occur
    tok, mx = oracle.greedy_tokens(logits)
    for r in range(50):
        best = 0
        for v in range(1, 13):
            if logits[r, v] > logits[r, best]:
                best = v
        assert tok[r] == best and mx[r] == logits[r, best]


def test_verify_head_designed_argmax():
    # one feature carries the row; W[v] peaks at v = t: logits = -(v - t)^2 + const after norm
    D, V = 8, 40
    W = np.zeros((V, D))
    v = np.arange(V)
    W[:, 0] = v
    W[:, 1] = -0.5 * v * v
    for t in (0, 7, 39):
        H = np.zeros((1, D))
        H[0, 0], H[0, 1] = float(t), 1.0       # logits ~ t v - v^2 / 2, maximal at v = t
        tok, _ = oracle.verify_head(H, np.ones(D), W, 0.0)
        assert tok[0] == t


def test_greedy_token_nan_logits_are_never_chosen():
    """A NaN logit is no candidate: it neither wins nor blocks a later maximum; a row of NaN has
    no candidate (token -1, best logit NaN); +inf and -inf are ordinary candidates."""
    nan, inf = np.nan, np.inf
    logits = np.array([[0.5, nan, 2.0, 1.0],          # NaN before the maximum
                       [nan, nan, nan, nan],          # no candidate
                       [nan, -inf, -inf, nan],        # only -inf candidates: the first one
                       [1.0, inf, nan, inf],          # +inf is the maximum, lowest index wins
                       [nan, -3.0, nan, -3.0],        # tie after a NaN
                       [7.0, nan, nan, nan]])         # maximum before the NaNs
    tok, mx = oracle.greedy_tokens(logits)
    assert tok.tolist() == [2, -1, 1, 1, 1, 0]
    assert mx[0] == 2.0 and np.isnan(mx[1]) and mx[2] == -inf and mx[3] == inf
    assert mx[4] == -3.0 and mx[5] == 7.0


def test_greedy_token_nan_brute_force():
    rng = np.random.default_rng(4)
    logits = np.round(rng.standard_normal((60, 9)), 1)
    logits[rng.random(logits.shape) < 0.3] = np.nan
    logits[5] = np.nan
    tok, mx = oracle.greedy_tokens(logits)
    for r in range(60):
        best = -1
        for v in range(9):
            x = logits[r, v]
            if x != x:                    # NaN: skipped
                continue
            if best < 0 or x > logits[r, best]:
                best = v
        assert tok[r] == best
        if best < 0:
            assert np.isnan(mx[r])
        else:
            assert mx[r] == logits[r, best]
