"""Pins of the ragged-batch oracle (SemKV Fig. 6 per prompt and per block;
Table 2, multi-turn).  The ragged oracle is the batch-of-one generation
oracle per sequence; these tests tie it to the batched generation oracle
(itself pinned elsewhere), to the counter invariants the pages fix (every
token is kept; every full block contributes exactly its top-r count) and to
hand-computed counts."""
import numpy as np
import pytest

import oracle as O

LAYERS, KV = 1, 2


def _tok(rng, n=None):
    shape = (LAYERS, KV, 128) if n is None else (LAYERS, KV, n, 128)
    return rng.standard_normal(shape).astype(np.float16)


def test_hand_counts():
    """Prompt of 300 at r = .25: k = floor(75.5) = 75.  Then 200 tokens with
    block 128: one full block (k = 32), 72 left; the flush ranks those 72
    with k = floor(18.5) = 18."""
    rng = np.random.default_rng(0)
    R = O.RaggedGeneration(2, LAYERS, KV, 6, 5, r=0.25, block=128)
    R.prompt(0, _tok(rng, 300), _tok(rng, 300), rng.random(300))
    assert R.counters(0) == (75, 225, 0, 300)
    assert R.counters(1) == (0, 0, 0, 0)
    for i in range(200):
        R.append(0, _tok(rng), _tok(rng), rng.random())
        if i == 127:
            assert R.counters(0) == (75 + 32, 225 + 96, 0, 428)
    assert R.counters(0) == (107, 321, 72, 500)
    R.flush(0)
    assert R.counters(0) == (125, 375, 0, 500)
    assert R.counters(1) == (0, 0, 0, 0)


def test_equals_batched_oracle_when_in_lockstep():
    """Sequences that see the same kinds of event at the same time give the
    pools of the batched generation oracle, sequence by sequence."""
    rng = np.random.default_rng(1)
    B, n, steps, r, block = 3, 90, 70, 0.35, 32
    K = rng.standard_normal((B, LAYERS, KV, n, 128)).astype(np.float16)
    V = rng.standard_normal((B, LAYERS, KV, n, 128)).astype(np.float16)
    s = rng.random((B, n)).astype(np.float32)
    G = O.GenerationCache(layers=LAYERS, kv_heads=KV, L_high=6, L_low=5, r=r, block=block, batch=B)
    R = O.RaggedGeneration(B, LAYERS, KV, 6, 5, r=r, block=block)
    G.prompt(K, V, s)
    for b in range(B):
        R.prompt(b, K[b], V[b], s[b])
    for _ in range(steps):
        kn = rng.standard_normal((B, LAYERS, KV, 128)).astype(np.float16)
        vn = rng.standard_normal((B, LAYERS, KV, 128)).astype(np.float16)
        sc = rng.random(B).astype(np.float32)
        G.append(kn, vn, sc)
        for b in range(B):
            R.append(b, kn[b], vn[b], sc[b])
    G.flush()
    for b in range(B):
        R.flush(b)
        p = R.pools(b)
        for f in ("codes_high", "codes_low", "meta_high", "meta_low", "tok_high", "tok_low"):
            assert np.array_equal(getattr(p, f)[0], getattr(G.pools, f)[b]), (b, f)


@pytest.mark.parametrize("seed", [2, 3])
def test_invariants_under_a_random_schedule(seed):
    """Random prompts, appends and flushes per sequence: every counter
    invariant holds after every event, every full block adds exactly
    topr(block) high rows, and the token indices of pools and tail cover each
    sequence's tokens exactly once."""
    rng = np.random.default_rng(seed)
    B, r, block = 3, 0.35, 20
    R = O.RaggedGeneration(B, LAYERS, KV, 6, 5, r=r, block=block)
    kb = O.topr_count(block, r)
    for _ in range(250):
        b = int(rng.integers(B))
        before = R.counters(b)
        ev = rng.random()
        if ev < 0.05 and before[2] == 0:
            n = int(rng.integers(1, 60))
            R.prompt(b, _tok(rng, n), _tok(rng, n), rng.random(n))
            k = O.topr_count(n, r)
            assert R.counters(b) == (before[0] + k, before[1] + n - k, 0, before[3] + n)
        elif ev < 0.12:
            R.flush(b)
            nt = before[2]
            k = O.topr_count(nt, r)
            assert R.counters(b) == (before[0] + k, before[1] + nt - k, 0, before[3])
        else:
            R.append(b, _tok(rng), _tok(rng), rng.random())
            nh, nl, nt, ntok = R.counters(b)
            if before[2] + 1 == block:
                assert (nh, nl, nt) == (before[0] + kb, before[1] + block - kb, 0)
            else:
                assert (nh, nl, nt) == (before[0], before[1], before[2] + 1)
            assert ntok == before[3] + 1
        for c in range(B):
            nh, nl, nt, ntok = R.counters(c)
            assert nh + nl + nt == ntok
            p = R.pools(c)
            toks = np.concatenate([p.tok_high[0], p.tok_low[0]])
            assert len(toks) == nh + nl
            assert np.array_equal(np.sort(toks), np.arange(nh + nl))   # the tail holds the rest


def test_sequences_are_independent():
    """Sequence 0's pools do not depend on what the other sequences do."""
    rng = np.random.default_rng(4)
    n = 50
    K0, V0, s0 = _tok(rng, n), _tok(rng, n), rng.random(n)
    toks = [(_tok(rng), _tok(rng), rng.random()) for _ in range(45)]
    out = []
    for other_steps in (0, 37):
        R = O.RaggedGeneration(2, LAYERS, KV, 6, 5, r=0.5, block=16)
        R.prompt(0, K0, V0, s0)
        R.prompt(1, _tok(rng, 7), _tok(rng, 7), rng.random(7))
        for i, (k, v, sc) in enumerate(toks):
            R.append(0, k, v, sc)
            if i < other_steps:
                R.append(1, _tok(rng), _tok(rng), rng.random())
        R.flush(0)
        out.append(R.pools(0))
    for f in ("codes_high", "codes_low", "meta_high", "meta_low", "tok_high", "tok_low"):
        assert np.array_equal(getattr(out[0], f), getattr(out[1], f)), f


def test_prompt_needs_empty_tail():
    rng = np.random.default_rng(5)
    R = O.RaggedGeneration(1, LAYERS, KV, 6, 5, r=0.5, block=16)
    R.append(0, _tok(rng), _tok(rng), 0.5)
    with pytest.raises(ValueError):
        R.prompt(0, _tok(rng, 3), _tok(rng, 3), rng.random(3))
