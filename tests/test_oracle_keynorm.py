"""Pins of the oracle's key-norm score (SemKV Fig. 2 and Table 3: a per-token
score from one model-internal indicator, key norm among them; read as the
sum of the key rows' Euclidean norms over a window of layers and every KV
head).  Each pin is a closed form or an exact construction, not the
oracle's formula typed again."""
import math

import numpy as np

import oracle as O


def test_closed_forms():
    B, layers, kv, n = 1, 3, 2, 5
    K = np.zeros((B, layers, kv, n, 128), np.float16)
    K[0, :, :, 0, :] = 0.5                        # norm 0.5 * sqrt(128) per row
    K[0, :, :, 1, 7] = -3.0                       # norm 3
    K[0, :, 0, 2, 0] = 3.0                        # a 3-4-5 triangle in head 0
    K[0, :, 0, 2, 99] = 4.0
    K[0, 1, 1, 3, :] = 0.0                        # token 3: zero everywhere
    K[0, 2, 1, 4, 5] = 2.0                        # token 4: one row only, in the last layer
    s = O.score_keynorm(K, 0, layers)
    assert s.shape == (1, n)
    assert math.isclose(s[0, 0], layers * kv * 0.5 * math.sqrt(128), rel_tol=1e-15)
    assert s[0, 1] == layers * kv * 3.0
    assert s[0, 2] == layers * 5.0
    assert s[0, 3] == 0.0
    assert s[0, 4] == 2.0
    # a window holds only its layers
    assert O.score_keynorm(K, 2, 1)[0, 4] == 2.0
    assert O.score_keynorm(K, 0, 2)[0, 4] == 0.0
    assert O.score_keynorm(K, 1, 2)[0, 2] == 2 * 5.0


def test_invariances_and_additivity():
    rng = np.random.default_rng(11)
    K = rng.standard_normal((2, 4, 3, 9, 128)).astype(np.float16)
    s = O.score_keynorm(K, 0, 4)
    # sign flips and permutations of the 128 dims keep every norm
    perm = rng.permutation(128)
    assert np.allclose(O.score_keynorm(-K[..., perm], 0, 4), s, rtol=1e-14)
    # scaling by a power of two scales the score exactly
    assert np.array_equal(O.score_keynorm((K.astype(np.float32) * 4).astype(np.float16), 0, 4), 4 * s)
    # the score of a window is the sum of its layers' scores
    per_layer = sum(O.score_keynorm(K, layer, 1) for layer in range(4))
    assert np.allclose(per_layer, s, rtol=1e-14)
    # sequences are scored independently
    assert np.array_equal(O.score_keynorm(K[1:], 0, 4)[0], s[1])


def test_brute_force_small():
    rng = np.random.default_rng(3)
    K = rng.standard_normal((1, 2, 2, 3, 128)).astype(np.float16)
    s = O.score_keynorm(K, 0, 2)
    for t in range(3):
        tot = 0.0
        for layer in range(2):
            for h in range(2):
                acc = 0.0
                for d in range(128):
                    acc += float(K[0, layer, h, t, d]) ** 2
                tot += math.sqrt(acc)
        assert math.isclose(s[0, t], tot, rel_tol=1e-13)
