"""Pins of the oracle's optional Hadamard rotation (SemKV Table 2 lists a
Hadamard rotation in the default quantizer; the matrix and its precision are
open on the pages: the oracle reads them as the normalized Sylvester H_128,
applied in float32 by index-bit butterflies).

As in test_oracle_pins.py, no check re-types the oracle's formulas: the matrix
is rebuilt by the Kronecker recursion, the transform is held to the float64
product within the float32 rounding bound and to closed forms, the codes to an
exact rational round-half-even, and the decode to attention computed on the
un-rotated values.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle as O


def sylvester(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.kron(np.array([[1.0, 1.0], [1.0, -1.0]]), h)
    return h


def test_hadamard_matrix_is_sylvester_and_orthogonal():
    H = O.hadamard128()
    assert np.array_equal(H * math.sqrt(128), sylvester(128))
    assert np.allclose(H @ H.T, np.eye(128), atol=1e-14)
    assert np.array_equal(H, H.T)


def test_rotation_close_to_matrix_product():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((200, 128)) * np.exp(rng.uniform(-6, 6, (200, 1)))).astype(np.float16)
    y = O.rotate_rows_f32(x).astype(np.float64)
    exact = x.astype(np.float64) @ O.hadamard128()
    # seven float32 butterfly stages (each partial sum is at most sum|x|) and one scaling
    bound = (8 * 2.0 ** -24) * np.abs(x.astype(np.float64)).sum(axis=1, keepdims=True)
    assert np.all(np.abs(y - exact) <= bound)


def test_rotation_closed_forms():
    e0 = np.zeros(128, np.float16)
    e0[0] = 1.0
    assert np.all(O.rotate_rows_f32(e0) == np.float32(1.0 / math.sqrt(128)))
    c = np.full(128, 0.75, np.float16)                    # sums of equal values are exact
    y = O.rotate_rows_f32(c)
    assert y[0] == np.float32(np.float32(96.0) * np.float32(1.0 / math.sqrt(128)))
    assert np.all(y[1:] == 0.0)
    e5 = np.zeros(128, np.float16)
    e5[5] = -2.0                                          # column 5 of H times -2
    y5 = O.rotate_rows_f32(e5).astype(np.float64)
    assert np.array_equal(y5, -2.0 * sylvester(128)[:, 5] * np.float64(np.float32(1.0 / math.sqrt(128))))


def test_fp16_floor_brute_force():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(500) * 10, rng.standard_normal(100) * 1e-6, [0.0, -0.0]])
    f = O.fp16_floor(v).astype(np.float64)
    assert np.all(f <= v)
    nxt = np.nextafter(O.fp16_floor(v), np.float16(np.inf)).astype(np.float64)
    assert np.all(nxt > v)


def rational_rne(num, s, L):
    """clamp(round-half-even(num / s), 0, L - 1) with exact rationals."""
    q = Fraction(num) / Fraction(s)
    f = math.floor(q)
    r = q - f
    c = f + (1 if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1) else 0)
    return min(max(c, 0), L - 1)


@pytest.mark.parametrize("L", [5, 6, 16, 255])
def test_rotated_quantizer_exact_rational(L):
    rng = np.random.default_rng(L)
    x = rng.standard_normal((12, 128))
    x[:, 3] *= 40.0                                       # an outlier channel
    x = x.astype(np.float16)
    codes, s16, m16 = O.quantize_rows_rotated(x, L)
    y = O.rotate_rows_f32(x).astype(np.float64)
    for r in range(x.shape[0]):
        lo = Fraction(float(m16[r]))
        mn = Fraction(float(y[r].min()))
        assert lo <= mn                                   # floor of the minimum, in fp16
        assert Fraction(float(np.nextafter(m16[r], np.float16(np.inf)))) > mn
        d = Fraction(float(y[r].max())) - lo
        s = Fraction(float(s16[r]))
        assert s * (L - 1) >= d                           # ceiling scale: no code clips
        below = np.nextafter(s16[r], np.float16(-np.inf))
        assert Fraction(float(below)) * (L - 1) < d
        for j in range(128):
            assert codes[r, j] == rational_rne(Fraction(float(y[r, j])) - lo, s, L)


def test_rotation_lowers_error_on_outlier_rows():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((64, 128))
    x[:, 7] *= 30.0                                       # K rows with one large channel
    x = x.astype(np.float16)
    x64 = x.astype(np.float64)
    for L in (5, 6):
        c, s, m = O.quantize_rows(x, L)
        plain = O.dequantize_rows(c, s, m)
        cr, sr, mr = O.quantize_rows_rotated(x, L)
        rot = O.dequantize_rows(cr, sr, mr) @ O.hadamard128()     # back to the row domain
        assert np.mean((rot - x64) ** 2) < 0.5 * np.mean((plain - x64) ** 2)


def test_rotated_decode_near_lossless_at_65536_levels():
    """With 65536 levels the rotated cache holds the rotated rows to about
    2^-16 of their range.  H is orthogonal and symmetric, so decode over it
    (query rotated exactly, output rotated back) must agree with plain
    attention of the query itself over the raw fp16 rows."""
    rng = np.random.default_rng(4)
    B, layers, kv, n, Hq = 1, 2, 2, 90, 8
    K = rng.standard_normal((B, layers, kv, n, 128)).astype(np.float16)
    V = rng.standard_normal((B, layers, kv, n, 128)).astype(np.float16)
    perm = np.stack([rng.permutation(n) for _ in range(B)]).astype(np.int32)
    pools = O.quantize_pack_cache(K, V, perm, 30, 65536, 65536, rotate=True)
    assert pools.rotate
    q = (rng.standard_normal((B, layers, Hq, 128)) / 11.3).astype(np.float16)
    got = O.decode_attention(q, pools, 1.0)
    for b in range(B):
        for layer in range(layers):
            for h in range(Hq):
                g = h // (Hq // kv)
                ref = O.attention(q[b, layer, h].astype(np.float64),
                                  K[b, layer, g].astype(np.float64),
                                  V[b, layer, g].astype(np.float64), 1.0)
                assert np.max(np.abs(got[b, layer, h] - ref)) <= 2e-4 * np.max(np.abs(ref))


def test_rotated_generation_near_lossless_at_65536_levels():
    """A rotated cache with generated tokens: pool rows (rotated, 65536
    levels) and fp16 tail rows (not quantized, so not rotated).  Decode must
    agree with one softmax of q over all the raw rows, pool and tail alike
    (the exact rotation of the query undoes the rows' rotation)."""
    rng = np.random.default_rng(8)
    B, layers, kv, Hq, n0, gen, block = 1, 1, 2, 8, 40, 21, 16
    g = O.GenerationCache(layers=layers, kv_heads=kv, L_high=65536, L_low=65536, r=0.5,
                          block=block, batch=B, rotate=True)
    K0 = rng.standard_normal((B, layers, kv, n0, 128)).astype(np.float16)
    V0 = rng.standard_normal((B, layers, kv, n0, 128)).astype(np.float16)
    g.prompt(K0, V0, rng.random((B, n0)).astype(np.float32))
    ks = rng.standard_normal((gen, B, layers, kv, 128)).astype(np.float16)
    vs = rng.standard_normal((gen, B, layers, kv, 128)).astype(np.float16)
    for i in range(gen):
        g.append(ks[i], vs[i], rng.random(B).astype(np.float32))
    assert g.pools.rotate and g.n_tail == gen - block
    q = (rng.standard_normal((B, layers, Hq, 128)) / 11.3).astype(np.float16)
    got = g.decode(q, 1.0)
    Kall = np.concatenate([K0, np.moveaxis(ks, 0, 3)], axis=3).astype(np.float64)
    Vall = np.concatenate([V0, np.moveaxis(vs, 0, 3)], axis=3).astype(np.float64)
    for h in range(Hq):
        gi = h // (Hq // kv)
        z = Kall[0, 0, gi] @ q[0, 0, h].astype(np.float64)
        p = np.exp(z - z.max())
        ref = (p / p.sum()) @ Vall[0, 0, gi]
        assert np.max(np.abs(got[0, 0, h] - ref)) <= 2e-4 * np.max(np.abs(ref))


def test_unrotated_decode_unchanged_by_tail_split():
    """Without rotation, pools and tail are one softmax over every row: the
    oracle's decode equals attention over the concatenated rows."""
    rng = np.random.default_rng(12)
    g = O.GenerationCache(layers=1, kv_heads=1, L_high=65536, L_low=65536, r=0.5, block=8, batch=1)
    K0 = rng.standard_normal((1, 1, 1, 10, 128)).astype(np.float16)
    V0 = rng.standard_normal((1, 1, 1, 10, 128)).astype(np.float16)
    g.prompt(K0, V0, rng.random((1, 10)).astype(np.float32))
    k1 = rng.standard_normal((1, 1, 1, 128)).astype(np.float16)
    v1 = rng.standard_normal((1, 1, 1, 128)).astype(np.float16)
    g.append(k1, v1, np.array([0.5], np.float32))
    q = (rng.standard_normal((1, 1, 4, 128)) / 11.3).astype(np.float16)
    got = g.decode(q, 1.0)
    Kall = np.concatenate([K0[0, 0, 0], k1[0, 0]], axis=0).astype(np.float64)
    Vall = np.concatenate([V0[0, 0, 0], v1[0, 0]], axis=0).astype(np.float64)
    for h in range(4):
        ref = O.attention(q[0, 0, h].astype(np.float64), Kall, Vall, 1.0)
        assert np.max(np.abs(got[0, 0, h] - ref)) <= 2e-4 * np.max(np.abs(ref))
