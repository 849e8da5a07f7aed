"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here re-types the oracle's own formulas: each check is a brute-force
enumeration, an exact rational computation (fractions.Fraction), a library
routine (numpy argsort, torch scaled_dot_product_attention), a closed-form
property, a hand-worked fixture (tests/golden/) or a figure printed on the
pages (tests/golden/page_figures.txt, each line citing its table/figure).
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from conftest import read_table

# ----------------------------------------------------------------- ranking


def ranks_before(s, i, j):
    """Token i precedes token j: higher score, equal scores by lower index,
    NaN below every number (open on the pages; our reading)."""
    a, b = float(s[i]), float(s[j])
    if math.isnan(a) and math.isnan(b):
        return i < j
    if math.isnan(a):
        return False
    if math.isnan(b):
        return True
    if a != b:
        return a > b
    return i < j


def brute_force_topk(s, k):
    """The unique k-subset H with every member ranking before every non-member."""
    n = len(s)
    hits = []
    for H in itertools.combinations(range(n), k):
        hs = set(H)
        if all(ranks_before(s, i, j) for i in hs for j in range(n) if j not in hs):
            hits.append(hs)
    assert len(hits) == 1
    return hits[0]


def _tie_rich_scores(rng, n):
    pool = np.array([0.0, -0.0, 1.0, 1.0, 2.5, -3.0, np.inf, -np.inf, np.nan, 0.5],
                    dtype=np.float32)
    return rng.choice(pool, size=n)


@pytest.mark.parametrize("seed", range(40))
def test_rank_brute_force_small(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 10))
    s = _tie_rich_scores(rng, n) if seed % 2 else rng.random(n).astype(np.float32)
    for k in range(n + 1):
        perm, mask = O.rank_topr(s, k)
        H = brute_force_topk(s, k)
        assert set(perm[:k].tolist()) == H
        # perm: H ascending, then the rest ascending, a permutation of 0..n-1
        assert perm[:k].tolist() == sorted(H)
        assert perm[k:].tolist() == sorted(set(range(n)) - H)
        for t in range(n):
            bit = (int(mask[t // 32]) >> (t % 32)) & 1
            assert bit == (t in H)


def test_rank_matches_stable_argsort():
    """Library routine: a stable descending argsort has the same top-k set
    when the scores hold no NaN."""
    rng = np.random.default_rng(5)
    for n in (1, 7, 100, 1000, 4099):
        s = rng.integers(0, 7, size=n).astype(np.float32)   # many ties
        for k in (0, 1, n // 3, n - 1, n):
            k = max(0, min(n, k))
            perm, _ = O.rank_topr(s, k)
            ref = np.argsort(-s, kind="stable")[:k]
            assert set(perm[:k].tolist()) == set(ref.tolist())


def test_rank_special_cases():
    s = np.full(70, 0.25, np.float32)
    perm, mask = O.rank_topr(s, 33)
    assert perm[:33].tolist() == list(range(33))          # all equal -> lowest indices
    assert mask.tolist() == [0xFFFFFFFF, 0x1, 0x0]
    perm, mask = O.rank_topr(s, 0)
    assert perm.tolist() == list(range(70)) and not mask.any()
    perm, mask = O.rank_topr(s, 70)
    assert perm.tolist() == list(range(70)) and mask.tolist() == [0xFFFFFFFF, 0xFFFFFFFF, 0x3F]
    # a NaN block ranks last; -0 and +0 tie and go by index
    s = np.array([np.nan, -0.0, 0.0, np.nan, -1.0], np.float32)
    assert O.rank_topr(s, 2)[0][:2].tolist() == [1, 2]
    assert O.rank_topr(s, 3)[0][:3].tolist() == [1, 2, 4]
    assert O.rank_topr(s, 4)[0][:4].tolist() == [0, 1, 2, 4]


def test_topr_count():
    # open on the pages; our reading: nearest integer, halves up
    assert O.topr_count(512, 0.25) == 128
    assert O.topr_count(32768, 0.5) == 16384
    assert O.topr_count(32768, 0.1) == 3277
    assert O.topr_count(32768, 0.9) == 29491
    assert O.topr_count(32768, 0.75) == 24576
    assert O.topr_count(128, 0.25) == 32
    assert O.topr_count(128, 0.35) == 45
    assert O.topr_count(2, 0.25) == 1
    assert O.topr_count(0, 0.5) == 0


# ------------------------------------------------------------ quantization


def fp16_ceil_exact(q: Fraction) -> Fraction:
    """Smallest fp16 >= q by exact rational comparison (walks numpy's fp16
    neighbours, compares with Fraction)."""
    h = np.float16(float(q))
    while Fraction(float(h)) < q:
        h = np.nextafter(h, np.float16(np.inf))
    while q > 0 and Fraction(float(np.nextafter(h, np.float16(-np.inf)))) >= q:
        h = np.nextafter(h, np.float16(-np.inf))
    return Fraction(float(h))


def exact_quantize(row16, L):
    """Quantizer definition evaluated in exact rational arithmetic."""
    xs = [Fraction(float(v)) for v in row16]
    lo, hi = min(xs), max(xs)
    if hi == lo:
        return [0] * len(xs), Fraction(0), lo
    s = fp16_ceil_exact((hi - lo) / (L - 1))
    codes = []
    for x in xs:
        t = (x - lo) / s
        c = t.numerator // t.denominator
        rem = t - c
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and c % 2 == 1):
            c += 1
        codes.append(min(max(c, 0), L - 1))
    return codes, s, lo


def test_hand_rows():
    for case, L, lead, fill, scale, mn, codes in read_table("hand_rows.txt"):
        L = int(L)
        lead = [float(v) for v in lead.split()]
        row = np.full(128, float(fill), np.float16)
        row[:len(lead)] = lead
        c, s, m = O.quantize_rows(row[None], L)
        assert float(s[0]) == float(scale), case
        assert float(m[0]) == float(mn), case
        want = [int(v) for v in codes.split()]
        assert c[0, :len(want)].tolist() == want, case


def _rows(rng, nrows, kind):
    if kind == "normal":
        x = rng.standard_normal((nrows, 128))
        x[:, :4] *= 10.0
    elif kind == "integers":        # exact ties are frequent
        x = rng.integers(-6, 7, size=(nrows, 128)).astype(np.float64)
    elif kind == "halves":
        x = rng.integers(-20, 21, size=(nrows, 128)) * 0.25
    elif kind == "subnormal":
        x = rng.integers(-300, 300, size=(nrows, 128)) * 2.0 ** -24
    elif kind == "wide":           # tiny and huge values in one row
        x = rng.standard_normal((nrows, 128)) * 1e-4
        x[:, 0] = 30000.0
        x[:, 1] = -2.0 ** -20
    else:
        raise ValueError(kind)
    return x.astype(np.float16)


@pytest.mark.parametrize("L", [3, 4, 5, 6, 7, 8, 16, 255, 65536])
@pytest.mark.parametrize("kind", ["normal", "integers", "halves", "subnormal", "wide"])
def test_quantize_exact_rational(L, kind):
    rng = np.random.default_rng(L * 31 + len(kind))
    rows = _rows(rng, 6, kind)
    c, s, m = O.quantize_rows(rows, L)
    for i in range(rows.shape[0]):
        codes, se, lo = exact_quantize(rows[i], L)
        assert Fraction(float(s[i])) == se
        assert Fraction(float(m[i])) == lo
        assert c[i].tolist() == codes


@pytest.mark.parametrize("L", [3, 4, 5, 6, 8, 16, 512])
def test_quantize_closed_forms(L):
    rng = np.random.default_rng(L)
    rows = np.concatenate([_rows(rng, 200, "normal"), _rows(rng, 50, "integers")])
    c, s, m = O.quantize_rows(rows, L)
    x = rows.astype(np.float64)
    xh = O.dequantize_rows(c, s, m)
    s64 = s.astype(np.float64)
    # reconstruction within half a step, everywhere
    assert np.all(np.abs(xh - x) <= s64[:, None] / 2)
    # the minimum reconstructs exactly and maps to 0; the maximum maps to L-1
    amin = x.argmin(axis=1)
    amax = x.argmax(axis=1)
    r = np.arange(rows.shape[0])
    assert np.all(c[r, amin] == 0) and np.all(xh[r, amin] == x[r, amin])
    assert np.all(c[r, amax] == L - 1)
    # alphabet is exactly {0 .. L-1}
    assert c.min() == 0 and c.max() == L - 1
    if L <= 16:
        assert set(np.unique(c).tolist()) == set(range(L))


def test_constant_row_exact():
    for L in (3, 5, 6, 65536):
        row = np.full((1, 128), -1.5, np.float16)
        c, s, m = O.quantize_rows(row, L)
        assert float(s[0]) == 0.0 and not c.any()
        assert np.all(O.dequantize_rows(c, s, m) == -1.5)


def test_signed_zero_minimum_stored_as_plus_zero():
    row = np.full((1, 128), 1.0, np.float16)
    row[0, 3] = -0.0
    row[0, 4] = 0.0
    c, s, m = O.quantize_rows(row, 6)
    assert O.fp16_bits(m)[0] == 0x0000
    assert c[0, 3] == 0 and c[0, 4] == 0


def test_L65536_round_trip_bounds():
    """At 65536 levels (our reading of a round trip) the affine step can be coarser than the
    fp16 spacing near 0, so the round trip is a bound, not bit equality."""
    rng = np.random.default_rng(3)
    rows = _rows(rng, 300, "normal")
    c, s, m = O.quantize_rows(rows, 65536)
    x = rows.astype(np.float64)
    xh = O.dequantize_rows(c, s, m)
    assert np.all(np.abs(xh - x) <= s.astype(np.float64)[:, None] / 2)
    span = x.max(axis=1) - x.min(axis=1)
    big = np.abs(x) >= span[:, None] / 32
    assert np.all(xh.astype(np.float16)[big] == rows[big])
    # rows spanning [0, 65504 * 2^-k] on the 2^-k grid: 65504/65535 lies
    # above the fp16 just below 1, so the scale is exactly 2^-k and the round
    # trip is exact
    for kexp in (0, 4, 9):
        grid = rng.integers(0, 65505, size=(40, 128)).astype(np.float16).astype(np.float64)
        grid = np.floor(grid)                                  # fp16 integers stay integers
        grid[:, 0], grid[:, 1] = 0.0, 65504.0
        grid = (grid * 2.0 ** -kexp).astype(np.float16)
        cg, sg, mg = O.quantize_rows(grid, 65536)
        assert np.all(sg.astype(np.float64) == 2.0 ** -kexp)
        assert np.all(O.dequantize_rows(cg, sg, mg) == grid.astype(np.float64))


# ----------------------------------------------------------------- packing


def test_row_bytes():
    want = {3: 26, 4: 32, 5: 38, 6: 43, 8: 48, 16: 64, 65536: 256, 7: 48, 100: 112}
    for L, R in want.items():
        assert O.row_bytes(L) == R


def test_hand_packing():
    for case, L, codes, R, bytes_ in read_table("hand_packing.txt"):
        L, R = int(L), int(R)
        c = np.zeros(128, np.int64)
        for item in codes.split():
            p, v = item.split(":")
            c[int(p)] = int(v)
        want = np.zeros(R, np.uint8)
        for item in bytes_.split():
            p, v = item.split(":")
            want[int(p)] = int(v)
        got = O.pack_rows(c[None], L)[0]
        assert got.shape == (R,), case
        assert got.tolist() == want.tolist(), case


def pack_bigint(codes, L, g, b):
    """Independent construction of the layout with one Python integer per row."""
    nf = -(-128 // g)
    stream = 0
    for f in range(nf):
        v = 0
        for i in range(g):
            pos = g * f + i
            v += (int(codes[pos]) if pos < 128 else 0) * L ** i
        assert v < 2 ** b
        stream |= v << (b * f)
    return list(stream.to_bytes(-(-nf * b // 8), "little"))


@pytest.mark.parametrize("L", [3, 4, 5, 6, 7, 8, 9, 16, 100, 1000, 65536])
def test_pack_bigint_and_roundtrip(L):
    rng = np.random.default_rng(L)
    codes = rng.integers(0, L, size=(20, 128))
    codes[0] = L - 1
    codes[1] = 0
    packed = O.pack_rows(codes, L)
    g, b = O.group_params(L)
    for i in range(codes.shape[0]):
        assert packed[i].tolist() == pack_bigint(codes[i], L, g, b)
    assert np.array_equal(O.unpack_rows(packed, L), codes)


def test_textbook_nibbles():
    rng = np.random.default_rng(0)
    c4 = rng.integers(0, 4, size=(8, 128))
    want4 = (c4[:, 0::4] | c4[:, 1::4] << 2 | c4[:, 2::4] << 4 | c4[:, 3::4] << 6)
    assert np.array_equal(O.pack_rows(c4, 4), want4.astype(np.uint8))
    c16 = rng.integers(0, 16, size=(8, 128))
    want16 = c16[:, 0::2] | c16[:, 1::2] << 4
    assert np.array_equal(O.pack_rows(c16, 16), want16.astype(np.uint8))


# -------------------------------------------------- the pages' arithmetic


def _rounds_to(x, value, digits):
    return round(x, digits) == round(value, digits)


def test_bit_grid(figures):
    for L in (2, 3, 4, 5, 6, 8):
        v, d, _ = figures[f"bits_grid_L{L}"]
        assert _rounds_to(math.log2(L), v, d)


def test_nominal_average(figures):
    v, d, _ = figures["semkv_avg_bits_r025"]
    n = 512
    k = O.topr_count(n, 0.25)
    assert _rounds_to(O.nominal_bits(k, n, 6, 5), v, d)
    assert abs(O.nominal_bits(k, n, 6, 5) - (0.25 * math.log2(6) + 0.75 * math.log2(5))) < 1e-12
    v, d, _ = figures["widened_gap_avg_r030"]
    assert _rounds_to(O.nominal_bits(30, 100, 8, 4), v, d)


def page_code_bits(L):
    """Code bits per value implied by the page's packing rates (Table 6):
    our field rate b/g, except 6 levels where the page packs 5 codes in 13
    bits (2.6)."""
    if L == 6:
        return 13 / 5
    g, b = O.group_params(L)
    return b / g


def test_code_and_effective_bits(figures):
    for L in (4, 5, 6, 8):
        v, d, _ = figures[f"code_bits_L{L}"]
        assert _rounds_to(page_code_bits(L), v, d)
    for L in (4, 5, 8):   # our field rate equals the page's exactly
        g, b = O.group_params(L)
        assert _rounds_to(b / g, figures[f"code_bits_L{L}"][0], 3)
    # 6 levels: 3 codes per byte costs the same 43 bytes per 128-value row as
    # the page's 5 codes per 13 bits
    assert O.row_bytes(6) == -(-(-(-128 // 5)) * 13 // 8) == 43
    for L in (4, 5):
        v, d, _ = figures[f"eff_bits_affine_L{L}"]
        assert _rounds_to(page_code_bits(L) + 32 / 128, v, d)   # two 16-bit scalars / row
    for L in (2, 3, 4, 5, 6, 8):
        v, d, _ = figures[f"eff_bits_tq_L{L}"]
        assert _rounds_to(page_code_bits(L) + 16 / 128, v, d)   # one 16-bit scalar / row


def test_compression_ratios(figures):
    for L in (4, 5, 6, 8):
        v, d, _ = figures[f"compression_uniform_L{L}"]
        assert _rounds_to(16 / (page_code_bits(L) + 0.25), v, d)
    semkv = 0.25 * page_code_bits(6) + 0.75 * page_code_bits(5) + 0.25
    v, d, _ = figures["compression_semkv_r025"]
    assert _rounds_to(16 / semkv, v, d)
    tq_code = 0.75 * page_code_bits(4) + 0.25 * page_code_bits(3)
    assert _rounds_to(tq_code, *figures["tq_r075_code_bits"][:2])
    assert _rounds_to(16 / (tq_code + 0.125), *figures["compression_tq_r075_L4L3"][:2])
    prune_bits = 16 * 0.25
    assert _rounds_to(prune_bits, *figures["prune_keep25_bits"][:2])
    assert _rounds_to(16 / prune_bits, *figures["prune_keep25_compression"][:2])
    v, d, _ = figures["prune_vs_semkv_footprint"]
    assert _rounds_to(figures["compression_semkv_r025"][0] / (16 / prune_bits), v, d)
    # this format's byte-rounded rows (43 + 4 and 38 + 4 bytes per row)
    fb = O.format_bits(128, 512, 6, 5)
    assert abs(fb - (128 * 47 + 384 * 42) * 8 / (128 * 512)) < 1e-12
    assert round(16 / fb, 2) == 5.92


# --------------------------------------------------------------- attention


def _small_cache(seed, B=1, layers=2, kv=2, n=40, Lh=6, Ll=5, r=0.25):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((B, layers, kv, n, 128)).astype(np.float16)
    V = rng.standard_normal((B, layers, kv, n, 128)).astype(np.float16)
    s = rng.random((B, n)).astype(np.float32)
    k = O.topr_count(n, r)
    perm, _ = O.rank_topr_batch(s, k)
    pools = O.quantize_pack_cache(K, V, perm, k, Lh, Ll)
    return K, V, s, perm, k, pools


def test_decode_matches_sdpa():
    B, layers, kv, Hq = 2, 2, 2, 8
    K, V, s, perm, k, pools = _small_cache(1, B=B, layers=layers, kv=kv)
    rng = np.random.default_rng(9)
    q = (rng.standard_normal((B, layers, Hq, 128)) / math.sqrt(128)).astype(np.float16)
    for sm in (1.0, 1 / math.sqrt(128)):
        out = O.decode_attention(q, pools, sm)
        for b in range(B):
            for layer in range(layers):
                kh = np.concatenate([O.dequantize_pool(pools.codes_high[b, layer], pools.meta_high[b, layer], 6),
                                     O.dequantize_pool(pools.codes_low[b, layer], pools.meta_low[b, layer], 5)],
                                    axis=2)                                   # [kv][2][n][128]
                keys = torch.tensor(kh[:, 0]).repeat_interleave(Hq // kv, dim=0)[None]
                vals = torch.tensor(kh[:, 1]).repeat_interleave(Hq // kv, dim=0)[None]
                qq = torch.tensor(q[b, layer].astype(np.float64))[None, :, None, :]
                ref = torch.nn.functional.scaled_dot_product_attention(qq, keys, vals, scale=sm)
                np.testing.assert_allclose(out[b, layer], ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)


def test_decode_special_cases():
    rng = np.random.default_rng(2)
    q = rng.standard_normal(128)
    v = rng.standard_normal((1, 128))
    assert np.allclose(O.attention(q, rng.standard_normal((1, 128)), v, 1.0), v[0])
    keys = np.tile(rng.standard_normal(128), (7, 1))          # equal logits
    vals = rng.standard_normal((7, 128))
    assert np.allclose(O.attention(q, keys, vals, 0.3), vals.mean(axis=0))
    keys = rng.standard_normal((50, 128))
    p = rng.permutation(50)
    assert np.allclose(O.attention(q, keys, vals.repeat(8, 0)[:50], 1.0),
                       O.attention(q, keys[p], vals.repeat(8, 0)[:50][p], 1.0))


def test_decode_L65536_close_to_fp16_cache():
    B, layers, kv, Hq, n = 1, 1, 2, 8, 64
    rng = np.random.default_rng(4)
    K = rng.standard_normal((B, layers, kv, n, 128)).astype(np.float16)
    V = rng.standard_normal((B, layers, kv, n, 128)).astype(np.float16)
    q = (rng.standard_normal((B, layers, Hq, 128)) / math.sqrt(128)).astype(np.float16)
    perm = np.tile(np.arange(n, dtype=np.int32), (B, 1))
    pools = O.quantize_pack_cache(K, V, perm, 16, 65536, 65536)
    out = O.decode_attention(q, pools, 1.0)
    for h in range(Hq):
        ref = O.attention(q[0, 0, h].astype(np.float64), K[0, 0, h // 4].astype(np.float64),
                          V[0, 0, h // 4].astype(np.float64), 1.0)
        assert np.max(np.abs(out[0, 0, h] - ref)) < 1e-4


def test_tail_rows_read_exactly():
    """A cache of tail rows only is plain attention over the fp16 rows."""
    rng = np.random.default_rng(6)
    gen = O.GenerationCache(layers=1, kv_heads=2, L_high=6, L_low=5, r=0.25, block=128, batch=1)
    ks = rng.standard_normal((10, 1, 1, 2, 128)).astype(np.float16)
    vs = rng.standard_normal((10, 1, 1, 2, 128)).astype(np.float16)
    for i in range(10):
        gen.append(ks[i], vs[i], rng.random(1))
    q = rng.standard_normal((1, 1, 8, 128)).astype(np.float16)
    out = gen.decode(q, 1.0)
    for h in range(8):
        ref = O.attention(q[0, 0, h].astype(np.float64), ks[:, 0, 0, h // 4].astype(np.float64),
                          vs[:, 0, 0, h // 4].astype(np.float64), 1.0)
        assert np.allclose(out[0, 0, h], ref, rtol=1e-13, atol=1e-13)


# -------------------------------------------------------------- generation


def test_generation_block_exact():
    """Counters preserve every token; each full block adds exactly k_b high
    rows; streaming equals ranking + quantizing each block on its own."""
    rng = np.random.default_rng(8)
    B, layers, kv, blk, r = 2, 1, 2, 16, 0.25
    gen = O.GenerationCache(layers=layers, kv_heads=kv, L_high=6, L_low=5, r=r, block=blk, batch=B)
    n0 = 20
    K0 = rng.standard_normal((B, layers, kv, n0, 128)).astype(np.float16)
    V0 = rng.standard_normal((B, layers, kv, n0, 128)).astype(np.float16)
    s0 = rng.random((B, n0)).astype(np.float32)
    gen.prompt(K0, V0, s0)
    steps = 3 * blk + 5
    ks = rng.standard_normal((steps, B, layers, kv, 128)).astype(np.float16)
    vs = rng.standard_normal((steps, B, layers, kv, 128)).astype(np.float16)
    ss = rng.random((steps, B)).astype(np.float32)
    kb = O.topr_count(blk, r)
    for i in range(steps):
        gen.append(ks[i], vs[i], ss[i])
        nh, nl = gen.pools.codes_high.shape[4], gen.pools.codes_low.shape[4]
        assert nh + nl + gen.n_tail == n0 + i + 1
        blocks = (i + 1) // blk
        assert nh == O.topr_count(n0, r) + blocks * kb
    gen.flush()
    assert gen.n_tail == 0
    # offline: prompt, then each block (and the residual) ranked on its own
    off_h, off_l = [], []
    pr = O.quantize_pack_cache(K0, V0, O.rank_topr_batch(s0, O.topr_count(n0, r))[0],
                               O.topr_count(n0, r), 6, 5)
    off_h.append(pr.codes_high), off_l.append(pr.codes_low)
    toks = [pr.tok_high], [pr.tok_low]
    for start in range(0, steps, blk):
        end = min(start + blk, steps)
        Kb = np.moveaxis(ks[start:end], 0, 3)
        Vb = np.moveaxis(vs[start:end], 0, 3)
        sb = ss[start:end].T
        kk = O.topr_count(end - start, r)
        pb = O.quantize_pack_cache(Kb, Vb, O.rank_topr_batch(sb, kk)[0], kk, 6, 5,
                                   token_base=n0 + start)
        off_h.append(pb.codes_high), off_l.append(pb.codes_low)
        toks[0].append(pb.tok_high), toks[1].append(pb.tok_low)
    assert np.array_equal(gen.pools.codes_high, np.concatenate(off_h, axis=4))
    assert np.array_equal(gen.pools.codes_low, np.concatenate(off_l, axis=4))
    assert np.array_equal(gen.pools.tok_high, np.concatenate(toks[0], axis=1))
    all_tok = np.sort(np.concatenate([gen.pools.tok_high, gen.pools.tok_low], axis=1), axis=1)
    assert np.array_equal(all_tok, np.tile(np.arange(n0 + steps), (B, 1)))   # nothing deleted


def test_realized_fraction_exact():
    """When r * block is an integer, the realized high fraction is exactly r."""
    gen = O.GenerationCache(layers=1, kv_heads=1, L_high=6, L_low=5, r=0.25, block=128, batch=1)
    rng = np.random.default_rng(0)
    for _ in range(256):
        gen.append(rng.standard_normal((1, 1, 1, 128)).astype(np.float16),
                   rng.standard_normal((1, 1, 1, 128)).astype(np.float16), rng.random(1))
    nh, nl = gen.pools.codes_high.shape[4], gen.pools.codes_low.shape[4]
    assert nh / (nh + nl) == 0.25
