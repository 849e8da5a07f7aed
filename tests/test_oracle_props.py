"""Property tests of the CPU oracle (randomised, CPU only).

Each property is checked with arithmetic that does not reuse the oracle's own
code path: exact rationals (fractions.Fraction, Python's round-half-even on
them), the pairwise characterisation of a top-k set, a big-integer rendering
of the packed bit stream, and invariances of softmax attention.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle as O

SET = settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])

# scores drawn from a small alphabet so that ties, signed zeros and NaNs are common
_ALPHABET = [0.0, -0.0, 1.0, -1.0, 0.5, 2.0, float("nan"), float("inf"), -float("inf")]


def _key_better(si, i, sj, j):
    """True iff token i ranks strictly ahead of token j (score desc, NaN last, index asc)."""
    ni, nj = math.isnan(si), math.isnan(sj)
    if ni != nj:
        return nj
    if not ni and si != sj:
        return si > sj
    return i < j


@SET
@given(st.lists(st.sampled_from(_ALPHABET), min_size=1, max_size=40), st.data())
def test_rank_pairwise_characterisation(vals, data):
    s = np.array(vals, dtype=np.float32)
    n = len(vals)
    k = data.draw(st.integers(0, n))
    perm, mask = O.rank_topr(s, k)
    assert sorted(perm.tolist()) == list(range(n))
    H = perm[:k].tolist()
    rest = perm[k:].tolist()
    assert H == sorted(H) and rest == sorted(rest)
    for i in H:
        for j in rest:
            assert _key_better(float(s[i]), i, float(s[j]), j)
    for t in range(n):
        assert bool((int(mask[t // 32]) >> (t % 32)) & 1) == (t in set(H))


def _fp16_ceil_exact(q: Fraction) -> Fraction:
    """Smallest fp16 >= q > 0, by walking the fp16 grid with exact rationals."""
    x = np.float16(float(q))
    while Fraction(float(x)) < q:
        x = np.nextafter(x, np.float16(np.inf))
    while True:
        y = np.nextafter(x, np.float16(-np.inf))
        if Fraction(float(y)) >= q:
            x = y
        else:
            return Fraction(float(x))


_rows = st.lists(st.floats(-300.0, 300.0, width=16, allow_subnormal=True), min_size=128,
                 max_size=128)


@SET
@given(_rows, st.sampled_from([3, 4, 5, 6, 7, 8, 13, 16, 100, 255, 4096]))
def test_quantize_exact_rationals(vals, L):
    x = np.array(vals, dtype=np.float16)
    codes, s16, m16 = O.quantize_rows(x[None, :], L)
    xs = [Fraction(float(v)) for v in x]
    m, M = min(xs), max(xs)
    assert Fraction(float(m16[0])) == m
    if M == m:
        assert float(s16[0]) == 0.0 and not codes.any()
        return
    s = _fp16_ceil_exact((M - m) / (L - 1))
    assert Fraction(float(s16[0])) == s
    for xi, ci in zip(xs, codes[0].tolist()):
        expect = min(max(round((xi - m) / s), 0), L - 1)   # round(): half to even, exact
        assert ci == expect
        assert abs(m + ci * s - xi) <= s / 2
    assert min(codes[0]) == 0


@SET
@given(st.integers(3, 300) | st.sampled_from([65536, 1000, 2048]), st.integers(0, 2**31 - 1))
def test_pack_bitstream_bigint(L, seed):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, L, size=(3, 128))
    packed = O.pack_rows(c, L)
    g, b = O.group_params(L)
    R = O.row_bytes(L)
    assert packed.shape == (3, R)
    nf = -(-128 // g)
    for row in range(3):
        padded = c[row].tolist() + [0] * (nf * g - 128)
        big = 0
        for j in range(nf):
            field = sum(padded[g * j + i] * L ** i for i in range(g))
            assert field < 2 ** b
            big |= field << (b * j)
        assert int.from_bytes(packed[row].tobytes(), "little") == big
    assert (O.unpack_rows(packed, L) == c).all()


@SET
@given(st.integers(0, 2**31 - 1), st.integers(1, 40))
def test_attention_invariances(seed, T):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(128)
    keys = rng.standard_normal((T, 128))
    vals = rng.standard_normal((T, 128))
    o = O.attention(q, keys, vals, 0.3)
    # a convex combination of the values
    assert (o <= vals.max(axis=0) + 1e-12).all() and (o >= vals.min(axis=0) - 1e-12).all()
    # token order does not matter
    p = rng.permutation(T)
    assert np.allclose(O.attention(q, keys[p], vals[p], 0.3), o, rtol=0, atol=1e-12)
    # adding one vector to every key shifts every logit equally
    w = rng.standard_normal(128)
    assert np.allclose(O.attention(q, keys + w, vals, 0.3), o, rtol=0, atol=1e-9)
    # sm_scale 0: the plain mean of the values
    assert np.allclose(O.attention(q, keys, vals, 0.0), vals.mean(axis=0), atol=1e-12)


@settings(max_examples=15, deadline=None)
@given(st.integers(0, 2**31 - 1), st.lists(st.integers(1, 9), min_size=1, max_size=8),
       st.sampled_from([0.25, 0.5, 0.35]))
def test_generation_counters_and_blocks(seed, chunks, r):
    rng = np.random.default_rng(seed)
    B, layers, kv, block = 2, 1, 2, 8
    gen = O.GenerationCache(layers=layers, kv_heads=kv, L_high=6, L_low=5, r=r, block=block,
                            batch=B)
    n0 = 11
    K = rng.standard_normal((B, layers, kv, n0, 128)).astype(np.float16)
    V = rng.standard_normal((B, layers, kv, n0, 128)).astype(np.float16)
    gen.prompt(K, V, rng.random((B, n0), dtype=np.float32))
    high_expect = O.topr_count(n0, r)
    total = n0
    for c in chunks:
        for _ in range(c):
            gen.append(rng.standard_normal((B, layers, kv, 128)).astype(np.float16),
                       rng.standard_normal((B, layers, kv, 128)).astype(np.float16),
                       rng.random(B, dtype=np.float32))
            total += 1
            if gen.n_tail == 0:
                high_expect += O.topr_count(block, r)
        nh = gen.pools.codes_high.shape[4]
        nl = gen.pools.codes_low.shape[4]
        assert nh + nl + gen.n_tail == total == gen.n_tokens
        assert nh == high_expect
    tail = gen.n_tail
    gen.flush()
    high_expect += O.topr_count(tail, r)
    assert gen.n_tail == 0
    assert gen.pools.codes_high.shape[4] == high_expect
    # every token index appears exactly once across both pools, per sequence
    for b in range(B):
        toks = np.concatenate([gen.pools.tok_high[b], gen.pools.tok_low[b]])
        assert sorted(toks.tolist()) == list(range(total))
