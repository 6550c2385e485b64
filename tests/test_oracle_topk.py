"""Pins for the oracle's top-k selection (CPU only): brute force by a full
numpy stable sort on every row, plus closed-form special cases."""
import numpy as np
import pytest

import oracle


def brute_topk(row: np.ndarray, p: int, k: int) -> np.ndarray:
    n = min(p, row.size - 1) + 1
    cand = row[:n].astype(np.float64)
    cand = np.where(cand == 0.0, 0.0, cand)           # -0 and +0 are one value
    order = np.argsort(-cand, kind="stable")            # desc score, asc index on ties
    chosen = np.sort(order[:k])
    out = np.full(k, -1, np.int32)
    out[: chosen.size] = chosen
    return out


@pytest.mark.parametrize("levels", [3, 50, None])
def test_matches_full_sort(rng, levels):
    B, T, L, k = 2, 5, 3000, 64
    if levels is None:
        scores = rng.standard_normal((B, T, L)).astype(np.float32)
    else:
        scores = rng.integers(0, levels, size=(B, T, L)).astype(np.float32) / 16
    pos = rng.integers(0, L, size=(B, T)).astype(np.int32)
    pos[0, 0] = 10        # fewer candidates than k
    pos[0, 1] = L - 1
    got = oracle.topk(scores, pos, k)
    for b in range(B):
        for t in range(T):
            np.testing.assert_array_equal(got[b, t], brute_topk(scores[b, t], pos[b, t], k))


def test_ignores_scores_after_position(rng):
    L, k = 100, 8
    s = np.zeros((1, 1, L), np.float32)
    s[0, 0, 50:] = 1e9       # beyond p: never candidates
    got = oracle.topk(s, np.array([[40]], np.int32), k)
    np.testing.assert_array_equal(got[0, 0], np.arange(8))


def test_all_equal_takes_lowest_positions():
    L, k = 5000, 2048
    s = np.full((1, 1, L), 3.0, np.float32)
    got = oracle.topk(s, np.array([[L - 1]], np.int32), k)
    np.testing.assert_array_equal(got[0, 0], np.arange(k))


def test_increasing_takes_last_positions():
    L, k = 5000, 2048
    s = np.arange(L, dtype=np.float32)[None, None]
    got = oracle.topk(s, np.array([[L - 1]], np.int32), k)
    np.testing.assert_array_equal(got[0, 0], np.arange(L - k, L))


def test_short_row_returns_all_visible():
    L, k = 3000, 2048
    s = np.random.default_rng(1).standard_normal((1, 1, L)).astype(np.float32)
    got = oracle.topk(s, np.array([[999]], np.int32), k)
    np.testing.assert_array_equal(got[0, 0, :1000], np.arange(1000))
    assert np.all(got[0, 0, 1000:] == -1)


def test_signed_zero_is_one_value():
    s = np.array([[[0.0, -0.0, 0.0, -0.0, 5.0]]], np.float32)
    got = oracle.topk(s, np.array([[4]], np.int32), 3)
    np.testing.assert_array_equal(got[0, 0], [0, 1, 4])


def test_negative_scores_and_neg_inf():
    s = np.array([[[-1.0, -np.inf, -3.0, -0.5, -np.inf]]], np.float32)
    got = oracle.topk(s, np.array([[4]], np.int32), 4)
    np.testing.assert_array_equal(got[0, 0], [0, 1, 2, 3])
