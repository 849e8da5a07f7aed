"""Pins of the hidden-state delta-norm score (SemKV Table 2's default
indicator; the formula is our reading): closed forms that a dropped term, a
wrong sign, a wrong axis or a missing square root would each break."""
import math

import numpy as np

import oracle as O


def test_pythagorean_updates():
    """Updates (3, 4), (5, 12), (8, 15), (0, 0) of one token: norms 5, 13, 17,
    0 -> score 35, exactly."""
    d = 64
    H = np.zeros((1, 5, 2, d), np.float16)
    steps = [(3, 4), (5, 12), (8, 15), (0, 0)]
    for j, (a, b) in enumerate(steps, start=1):
        H[0, j] = H[0, j - 1]
        H[0, j, 0, 7] += a
        H[0, j, 0, 40] -= b
    s = O.score_hidden_delta(H)
    assert s[0, 0] == 35.0
    assert s[0, 1] == 0.0                      # a token whose states never change


def test_arithmetic_progression():
    """h_j = h_0 + j c: every update is c, so the score is S ||c||."""
    rng = np.random.default_rng(0)
    d, S = 128, 4
    c = rng.integers(-4, 5, size=d).astype(np.float64) / 4          # exact in fp16
    h0 = rng.integers(-64, 64, size=d).astype(np.float64) / 8
    H = np.stack([h0 + j * c for j in range(S + 1)])[None, :, None, :].astype(np.float16)
    assert np.isclose(O.score_hidden_delta(H)[0, 0], S * math.sqrt(float(np.sum(c * c))),
                      rtol=1e-15)


def test_single_update_is_a_library_norm():
    """One layer (S = 1): the score is numpy's 2-norm of the difference."""
    rng = np.random.default_rng(1)
    H = rng.standard_normal((2, 2, 9, 96)).astype(np.float16)
    want = np.linalg.norm(H[:, 1].astype(np.float64) - H[:, 0].astype(np.float64), axis=-1)
    assert np.allclose(O.score_hidden_delta(H), want, rtol=1e-14, atol=0)


def test_symmetries():
    """Reversing the layer order, negating every state or adding one vector
    to every state leaves the score unchanged; scaling by 2 doubles it."""
    rng = np.random.default_rng(2)
    H = (rng.integers(-512, 512, size=(1, 5, 6, 64)) / 16).astype(np.float16)   # exact, and so are the shifts below
    s = O.score_hidden_delta(H)
    assert np.allclose(O.score_hidden_delta(H[:, ::-1]), s, rtol=1e-14)
    assert np.allclose(O.score_hidden_delta(-H), s, rtol=0, atol=0)
    shift = (rng.integers(-8, 8, size=64) / 2).astype(np.float16)
    Hs = H.astype(np.float64) + shift
    assert np.array_equal(Hs.astype(np.float16).astype(np.float64), Hs)   # still exact in fp16
    assert np.allclose(O.score_hidden_delta(Hs.astype(np.float16)), s, rtol=1e-14)
    assert np.allclose(O.score_hidden_delta((H.astype(np.float64) * 2).astype(np.float16)), 2 * s,
                       rtol=1e-15)


def test_each_layer_counts_once():
    """Triangle inequality: going from h_0 to h_S through the S updates is at
    least the direct distance; equal when the updates are parallel."""
    rng = np.random.default_rng(3)
    H = rng.standard_normal((1, 5, 20, 32)).astype(np.float16)
    direct = np.linalg.norm(H[0, 4].astype(np.float64) - H[0, 0].astype(np.float64), axis=-1)
    assert np.all(O.score_hidden_delta(H)[0] >= direct * (1 - 1e-14))
