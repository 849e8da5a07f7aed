"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Sizes are small enough for the oracle to finish in seconds but span several
64-row tiles and ragged tails.  Rank, codes, packed bytes, meta and the
slot->token maps must be bit-exact; decode attention within 2e-3 abs/rel.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity_helpers import assert_attention_close, assert_pools_equal, cap16, gpu_pools, to_dev

pytestmark = pytest.mark.gpu

sk = pytest.importorskip("kv_cache_mixed_top_amd.semkv")


def _print(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ rank

def _rank_gpu(scores, k):
    s = to_dev(scores.astype(np.float32))
    B, n = scores.shape
    perm = torch.empty((B, n), dtype=torch.int32, device="cuda")
    mask = torch.empty((B, (n + 31) // 32), dtype=torch.int32, device="cuda")
    sk.semkv_rank_topr(s, k, perm, mask)
    sk.semkv_sync_check()
    return perm.cpu().numpy(), mask.cpu().numpy().view(np.uint32)


def _check_rank(scores, k, what):
    perm, mask = _rank_gpu(scores, k)
    wp, wm = O.rank_topr_batch(scores, k)
    assert np.array_equal(perm, wp), f"{what}: perm differs"
    assert np.array_equal(mask, wm), f"{what}: mask differs"


@pytest.mark.parametrize("n", [1, 2, 31, 32, 33, 64, 100, 127, 128, 129, 200, 1000, 1024, 1025,
                               4099, 32767, 32768, 32769, 40000])
def test_rank_random(n):
    _print("rank random n", n)
    rng = np.random.default_rng(n)
    s = rng.random((3, n)).astype(np.float32)
    for r in (0.0, 0.1, 0.25, 0.5, 1.0):
        _check_rank(s, O.topr_count(n, r), f"n={n} r={r}")


@pytest.mark.parametrize("n", [5, 77, 128, 300, 5000, 32768, 33000])
def test_rank_ties_nan_signed_zero(n):
    _print("rank ties n", n)
    rng = np.random.default_rng(7 + n)
    pool = np.array([0.0, -0.0, 1.0, 2.5, -3.0, np.inf, -np.inf, np.nan, 0.5, 1e-30],
                    dtype=np.float32)
    s = rng.choice(pool, size=(2, n))
    s[1, :] = 0.25                                   # all equal
    for k in sorted({0, 1, n // 7, n // 2, n - 1, n}):
        _check_rank(s, k, f"ties n={n} k={k}")


def test_rank_tiny_config():
    w = W.WORKLOADS["tiny"]
    inp = W.make_inputs_np(w)
    _check_rank(inp["scores"], O.topr_count(w.n, w.r), "tiny")


# ------------------------------------------------------------------ quantize + pack

def _quantize_case(K, V, scores, r, Lh, Ll, what, q_heads=None, max_decode_layers=None):
    B, layers, kv, n, _ = K.shape
    k = O.topr_count(n, r)
    cache = sk.SemKVCache(B, layers, kv, kv * 4 if q_heads is None else q_heads, Lh, Ll, cap16(k),
                          cap16(n - k), block=128, max_decode_layers=max_decode_layers, max_tokens=n)
    Kd, Vd = to_dev(K), to_dev(V)
    perm = torch.empty((B, n), dtype=torch.int32, device="cuda")
    sk.semkv_rank_topr(to_dev(scores), k, perm)
    sk.semkv_quantize_pack(cache, Kd, Vd, perm, k)
    sk.semkv_sync_check()
    assert (cache.n_high, cache.n_low, cache.n_tokens) == (k, n - k, n)
    wp, _ = O.rank_topr_batch(scores, k)
    assert np.array_equal(perm.cpu().numpy(), wp), what
    op = O.quantize_pack_cache(K, V, wp, k, Lh, Ll)
    assert_pools_equal(gpu_pools(cache, sk), op, what)
    return cache, op


def _kv(rng, B, layers, kv, n, kind="normal"):
    shape = (B, layers, kv, n, 128)
    if kind == "normal":
        K = rng.standard_normal(shape)
        K[..., :4] *= 10.0
        V = rng.standard_normal(shape)
    elif kind == "integers":
        K = rng.integers(-6, 7, size=shape).astype(np.float64)
        V = rng.integers(-3, 4, size=shape) * 0.5
    elif kind == "mixed":
        K = rng.standard_normal(shape)
        K[..., 5, :] = 1.5                                    # constant rows
        K[..., 6, :] = rng.integers(-300, 300, size=K[..., 6, :].shape) * 2.0 ** -24
        K[..., 7, :] = rng.standard_normal(K[..., 7, :].shape) * 1e-4
        K[..., 7, 0] = 30000.0
        V = rng.standard_normal(shape) * 1e-3
        V[..., 3, :] = -0.0
        V[..., 3, 9] = 0.0
    else:
        raise ValueError(kind)
    return K.astype(np.float16), V.astype(np.float16)


def test_quantize_tiny_config():
    w = W.WORKLOADS["tiny"]
    inp = W.make_inputs_np(w)
    _print("quantize tiny")
    _quantize_case(inp["K"], inp["V"], inp["scores"], w.r, 6, 5, "tiny")


@pytest.mark.parametrize("Lh,Ll", [(6, 5), (5, 4), (8, 6), (4, 3), (16, 8), (65536, 7),
                                   (6, 6), (255, 100)])
@pytest.mark.parametrize("kind", ["normal", "integers", "mixed"])
def test_quantize_levels(Lh, Ll, kind):
    _print("quantize", Lh, Ll, kind)
    rng = np.random.default_rng(Lh * 7 + Ll)
    B, layers, kv, n = 2, 2, 2, 203                    # 4 tiles with a ragged tail
    K, V = _kv(rng, B, layers, kv, n, kind)
    s = rng.random((B, n)).astype(np.float32)
    for r in (0.25, 0.5):
        _quantize_case(K, V, s, r, Lh, Ll, f"L=({Lh},{Ll}) {kind} r={r}")


@pytest.mark.parametrize("r", [0.0, 1.0])
def test_quantize_single_pool(r):
    _print("quantize single pool r", r)
    rng = np.random.default_rng(11)
    K, V = _kv(rng, 1, 1, 3, 130)
    s = rng.random((1, 130)).astype(np.float32)
    _quantize_case(K, V, s, r, 6, 6 if r == 1.0 else 5, f"r={r}")


def test_quantize_strided_input_and_append_offset():
    """K/V as a strided view (token-major storage) and two prompt calls
    filling the pools back to back at unaligned row offsets."""
    _print("quantize strided")
    rng = np.random.default_rng(12)
    B, layers, kv = 1, 2, 2
    n1, n2 = 37, 70
    base1 = rng.standard_normal((B, n1, layers, kv, 128)).astype(np.float16)
    base2 = rng.standard_normal((B, n2, layers, kv, 128)).astype(np.float16)
    s1 = rng.random((B, n1)).astype(np.float32)
    s2 = rng.random((B, n2)).astype(np.float32)
    k1, k2 = O.topr_count(n1, 0.3), O.topr_count(n2, 0.3)
    cache = sk.SemKVCache(B, layers, kv, kv, 6, 5, cap16(k1 + k2), cap16(n1 + n2 - k1 - k2))
    pools = []
    base_tok = 0
    for base, s, n, k in ((base1, s1, n1, k1), (base2, s2, n2, k2)):
        dev = to_dev(base).permute(0, 2, 3, 1, 4)        # [B][layers][kv][n][128] strided view
        perm = torch.empty((B, n), dtype=torch.int32, device="cuda")
        sk.semkv_rank_topr(to_dev(s), k, perm)
        cache.c.n_tail = 0
        sk.semkv_quantize_pack(cache, dev, dev, perm, k)   # V = K: same rows twice
        Kn = np.moveaxis(base, 1, 3)
        wp, _ = O.rank_topr_batch(s, k)
        pools.append(O.quantize_pack_cache(Kn, Kn, wp, k, 6, 5, token_base=base_tok))
        base_tok += n
    sk.semkv_sync_check()
    cat = O.Pools(6, 5, *[np.concatenate([getattr(p, f) for p in pools], axis=4 if "tok" not in f else 1)
                          for f in ("codes_high", "meta_high", "tok_high", "codes_low", "meta_low",
                                    "tok_low")])
    assert_pools_equal(gpu_pools(cache, sk), cat, "two prompts")


# ------------------------------------------------------------------ decode

def _decode_case(B, layers, kv, Hq, n, r, Lh, Ll, sm, seed, nl=None, layer0=0):
    rng = np.random.default_rng(seed)
    K, V = _kv(rng, B, layers, kv, n)
    s = rng.random((B, n)).astype(np.float32)
    nl = layers if nl is None else nl
    # the cache is built for the requested query head count and layer window
    cache, op = _quantize_case(K, V, s, r, Lh, Ll, f"decode setup seed={seed}", q_heads=Hq,
                               max_decode_layers=nl)
    q = (rng.standard_normal((B, nl, Hq, 128)) / math.sqrt(128)).astype(np.float16)
    out = torch.empty((B, nl, Hq, 128), dtype=torch.float32, device="cuda")
    sk.semkv_decode_attn(cache, to_dev(q), out, layer0=layer0, sm_scale=sm)
    sk.semkv_sync_check()
    ref = O.decode_attention(q, op, sm, layer0=layer0)
    return assert_attention_close(out.cpu().numpy(), ref, f"decode seed={seed}")


def test_decode_tiny_config():
    w = W.WORKLOADS["tiny"]
    inp = W.make_inputs_np(w)
    _print("decode tiny")
    cache, op = _quantize_case(inp["K"], inp["V"], inp["scores"], w.r, 6, 5, "tiny")
    q = inp["q"][0]
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    sk.semkv_decode_attn(cache, to_dev(q), out, sm_scale=w.sm_scale)
    sk.semkv_sync_check()
    assert_attention_close(out.cpu().numpy(), O.decode_attention(q, op, w.sm_scale), "tiny")


@pytest.mark.parametrize("case", [
    dict(B=1, layers=2, kv=2, Hq=8, n=300, r=0.5, Lh=6, Ll=5, sm=1.0),
    dict(B=2, layers=1, kv=4, Hq=4, n=257, r=0.25, Lh=6, Ll=5, sm=1 / math.sqrt(128)),
    dict(B=1, layers=3, kv=1, Hq=8, n=1500, r=0.1, Lh=8, Ll=4, sm=1.0),
    dict(B=1, layers=2, kv=2, Hq=2, n=90, r=0.75, Lh=16, Ll=3, sm=1.0),
    dict(B=1, layers=4, kv=2, Hq=8, n=200, r=0.5, Lh=6, Ll=5, sm=1.0, nl=2, layer0=1),
    dict(B=1, layers=1, kv=2, Hq=8, n=2500, r=0.9, Lh=65536, Ll=5, sm=1.0),
])
def test_decode_configs(case):
    _print("decode", case)
    _decode_case(seed=len(str(case)), **case)


# One sequence, one layer and 2 KV heads take the shortest chunks (256 rows),
# so the chunk count per head grows with n and each merge form runs: one wave
# per KV head (<= 8 and <= 16 chunks), one workgroup per query head (<= 32),
# and four chunk groups per query head (more).
@pytest.mark.parametrize("n", [500, 2500, 6000, 10000])
def test_decode_merge_chunk_counts(n):
    _print("decode merge chunks", n)
    _decode_case(B=1, layers=1, kv=2, Hq=8, n=n, r=0.5, Lh=6, Ll=5, sm=1.0, seed=n)


def test_decode_partials_merge_equals_fused():
    _print("decode partials+merge")
    rng = np.random.default_rng(3)
    B, layers, kv, n = 1, 2, 2, 700
    K, V = _kv(rng, B, layers, kv, n)
    s = rng.random((B, n)).astype(np.float32)
    cache, op = _quantize_case(K, V, s, 0.5, 6, 5, "pm")
    q = to_dev((rng.standard_normal((B, layers, 8, 128)) / 11.3).astype(np.float16))
    a = torch.empty((B, layers, 8, 128), dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    sk.semkv_decode_attn(cache, q, a)
    sk.semkv_decode_partials(cache, q)
    sk.semkv_decode_merge(cache, b)
    sk.semkv_sync_check()
    assert torch.equal(a, b)
    # determinism: same inputs, identical outputs
    sk.semkv_decode_attn(cache, q, b)
    sk.semkv_sync_check()
    assert torch.equal(a, b)


def test_decode_per_layer_graph_replay():
    """Per-layer partials + merge captured once in a HIP graph: every replay,
    with eager work and synchronisation between replays and a new query
    copied into the captured buffer, equals the same calls issued eagerly."""
    _print("decode per-layer graph")
    rng = np.random.default_rng(17)
    B, layers, kv, n = 1, 3, 2, 700
    K, V = _kv(rng, B, layers, kv, n)
    s = rng.random((B, n)).astype(np.float32)
    cache, op = _quantize_case(K, V, s, 0.5, 6, 5, "graph")
    qs = [(rng.standard_normal((B, layers, 8, 128)) / 11.3).astype(np.float16) for _ in range(3)]
    qbuf = to_dev(qs[0])
    out_g = torch.empty((B, layers, 8, 128), dtype=torch.float32, device="cuda")
    out_e = torch.empty_like(out_g)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()

    def per_layer(out, stream):
        for layer in range(layers):
            sk.semkv_decode_partials(cache, qbuf[:, layer:layer + 1], layer0=layer, stream=stream)
            sk.semkv_decode_merge(cache, out[:, layer:layer + 1], stream=stream)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        per_layer(out_g, side)
    for i, q in enumerate(qs + qs[:1]):
        qbuf.copy_(to_dev(q))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        per_layer(out_e, None)                       # eager, on the default stream
        sk.semkv_sync_check()
        assert torch.equal(out_g, out_e), f"replay {i}"
        assert_attention_close(out_g.cpu().numpy(), O.decode_attention(q, op, 1.0), f"replay {i}")


# ------------------------------------------------------------------ generation

@pytest.mark.parametrize("block,steps,r", [(128, 300, 0.25), (16, 53, 0.35), (128, 128, 0.5),
                                           (512, 300, 0.25)])
def test_generation_block_exact(block, steps, r):
    _print("generation", block, steps, r)
    rng = np.random.default_rng(block + steps)
    B, layers, kv, Hq, n0 = 2, 2, 2, 8, 150
    K0, V0 = _kv(rng, B, layers, kv, n0)
    s0 = rng.random((B, n0)).astype(np.float32)
    k0 = O.topr_count(n0, r)
    tot = n0 + steps
    cache = sk.SemKVCache(B, layers, kv, Hq, 6, 5, cap16(tot), cap16(tot), block=block,
                          max_tokens=tot + block)
    perm = torch.empty((B, n0), dtype=torch.int32, device="cuda")
    sk.semkv_rank_topr(to_dev(s0), k0, perm)
    sk.semkv_quantize_pack(cache, to_dev(K0), to_dev(V0), perm, k0)
    ref = O.GenerationCache(layers=layers, kv_heads=kv, L_high=6, L_low=5, r=r, block=block,
                            batch=B)
    ref.prompt(K0, V0, s0)
    ks = rng.standard_normal((steps, B, layers, kv, 128)).astype(np.float16)
    vs = rng.standard_normal((steps, B, layers, kv, 128)).astype(np.float16)
    ss = rng.random((steps, B)).astype(np.float32)
    out = torch.empty((B, layers, Hq, 128), dtype=torch.float32, device="cuda")
    # tails of 1, 16, 17 and block - 1 rows (the largest a decode sees: the
    # folded tail path's 16-row groups full, ragged and all present), none,
    # and the last step's
    check_at = {0, 15, 16, block - 2, block - 1, block, steps - 1}
    for i in range(steps):
        kd = to_dev(ks[i][:, :, :, None, :])
        vd = to_dev(vs[i][:, :, :, None, :])
        sd = to_dev(ss[i][:, None])
        sk.semkv_append_block(cache, kd, vd, sd, r)
        ref.append(ks[i], vs[i], ss[i])
        assert cache.n_tail == ref.n_tail
        assert cache.n_high + cache.n_low + cache.n_tail == n0 + i + 1
        if i in check_at:
            q = (rng.standard_normal((B, layers, Hq, 128)) / math.sqrt(128)).astype(np.float16)
            sk.semkv_decode_attn(cache, to_dev(q), out)
            sk.semkv_sync_check()
            assert_attention_close(out.cpu().numpy(), ref.decode(q, 1.0), f"gen step {i}")
    sk.semkv_append_block(cache, None, None, None, r, flush=True)
    ref.flush()
    sk.semkv_sync_check()
    assert cache.n_tail == 0
    assert_pools_equal(gpu_pools(cache, sk), ref.pools, "after flush")


def test_multi_turn():
    """Two turns of prompt + generation (SemKV Fig. 6; the multi-turn setting
    uses r = 0.35): each prompt is ranked and quantized as a whole, each
    turn's generated tokens block by block, the residual block at the turn's
    end (flush); a prompt is refused while the tail holds tokens."""
    _print("multi-turn")
    rng = np.random.default_rng(35)
    B, layers, kv, Hq, block, r = 2, 2, 2, 8, 128, 0.35
    turns = [(150, 170), (90, 60)]                 # (prompt tokens, generated tokens)
    tot = sum(a + b for a, b in turns)
    cache = sk.SemKVCache(B, layers, kv, Hq, 6, 5, cap16(tot), cap16(tot), block=block,
                          max_tokens=tot + block)
    ref = O.GenerationCache(layers=layers, kv_heads=kv, L_high=6, L_low=5, r=r, block=block,
                            batch=B)
    out = torch.empty((B, layers, Hq, 128), dtype=torch.float32, device="cuda")
    for t_i, (n_p, n_g) in enumerate(turns):
        K, V = _kv(rng, B, layers, kv, n_p)
        s = rng.random((B, n_p)).astype(np.float32)
        k = O.topr_count(n_p, r)
        perm = torch.empty((B, n_p), dtype=torch.int32, device="cuda")
        sk.semkv_rank_topr(to_dev(s), k, perm)
        sk.semkv_quantize_pack(cache, to_dev(K), to_dev(V), perm, k)
        ref.prompt(K, V, s)
        ks = rng.standard_normal((B, layers, kv, n_g, 128)).astype(np.float16)
        vs = rng.standard_normal((B, layers, kv, n_g, 128)).astype(np.float16)
        ss = rng.random((B, n_g)).astype(np.float32)
        sk.semkv_append_block(cache, to_dev(ks), to_dev(vs), to_dev(ss), r)
        for i in range(n_g):
            ref.append(ks[:, :, :, i], vs[:, :, :, i], ss[:, i])
        assert cache.n_tail == ref.n_tail > 0
        if t_i == 0:                               # a prompt needs an empty tail
            with pytest.raises(sk.SemKVError):
                sk.semkv_quantize_pack(cache, to_dev(K), to_dev(V), perm, k)
        q = (rng.standard_normal((B, layers, Hq, 128)) / math.sqrt(128)).astype(np.float16)
        sk.semkv_decode_attn(cache, to_dev(q), out)
        sk.semkv_sync_check()
        assert_attention_close(out.cpu().numpy(), ref.decode(q, 1.0), f"turn {t_i} before flush")
        sk.semkv_append_block(cache, None, None, None, r, flush=True)
        ref.flush()
        sk.semkv_sync_check()
        assert cache.n_tail == 0 and cache.n_tokens == ref.n_tokens
        assert_pools_equal(gpu_pools(cache, sk), ref.pools, f"turn {t_i} after flush")
    q = (rng.standard_normal((B, layers, Hq, 128)) / math.sqrt(128)).astype(np.float16)
    sk.semkv_decode_attn(cache, to_dev(q), out)
    sk.semkv_sync_check()
    assert_attention_close(out.cpu().numpy(), ref.decode(q, 1.0), "after both turns")


def test_append_many_tokens_one_call():
    """t_new larger than a block: the call fills, quantizes and refills."""
    _print("append many")
    rng = np.random.default_rng(21)
    B, layers, kv, block, r = 1, 1, 2, 16, 0.25
    cache = sk.SemKVCache(B, layers, kv, 8, 6, 5, 64, 64, block=block)
    ref = O.GenerationCache(layers=layers, kv_heads=kv, L_high=6, L_low=5, r=r, block=block,
                            batch=B)
    t = 45
    K = rng.standard_normal((B, layers, kv, t, 128)).astype(np.float16)
    V = rng.standard_normal((B, layers, kv, t, 128)).astype(np.float16)
    s = rng.random((B, t)).astype(np.float32)
    sk.semkv_append_block(cache, to_dev(K), to_dev(V), to_dev(s), r, flush=True)
    for i in range(t):
        ref.append(K[:, :, :, i], V[:, :, :, i], s[:, i])
    ref.flush()
    sk.semkv_sync_check()
    assert_pools_equal(gpu_pools(cache, sk), ref.pools, "append many")


def test_checkpoint_roundtrip():
    _print("checkpoint")
    rng = np.random.default_rng(5)
    B, layers, kv, n = 1, 2, 2, 100
    K, V = _kv(rng, B, layers, kv, n)
    s = rng.random((B, n)).astype(np.float32)
    cache, _ = _quantize_case(K, V, s, 0.5, 6, 5, "ckpt")
    q = to_dev((rng.standard_normal((B, layers, 8, 128)) / 11.3).astype(np.float16))
    a = torch.empty((B, layers, 8, 128), dtype=torch.float32, device="cuda")
    sk.semkv_decode_attn(cache, q, a)
    state = cache.state_dict()
    other = sk.SemKVCache(B, layers, kv, 8, 6, 5, cache.geom.cap_high, cache.geom.cap_low)
    other.load_state_dict(state)
    b = torch.empty_like(a)
    sk.semkv_decode_attn(other, q, b)
    sk.semkv_sync_check()
    assert torch.equal(a, b)


# ------------------------------------------------------------------ matrix-core decode path
# Pools of 3, 4, 5, 6, 8 and 16 levels (any pair with L_high >= L_low) with 4 query
# heads per KV head take the MFMA kernel; these cases cover several 64-row
# tiles per chunk, ragged last tiles, empty pools, constant / tiny / wide rows
# and heavy-tailed V.

@pytest.mark.parametrize("n,r,kind", [
    (1, 0.5, "normal"), (63, 0.5, "normal"), (64, 0.25, "normal"), (65, 0.75, "normal"),
    (130, 0.5, "mixed"), (1000, 0.1, "normal"), (3000, 0.5, "mixed"), (5000, 0.9, "normal"),
    (700, 0.0, "normal"), (700, 1.0, "normal"), (2049, 0.5, "studentt"),
])
def test_decode_mfma_shapes(n, r, kind):
    _print("decode mfma", n, r, kind)
    rng = np.random.default_rng(n * 3 + int(r * 10))
    B, layers, kv, Hq = 2, 2, 2, 8
    if kind == "studentt":
        K, _ = _kv(rng, B, layers, kv, n)
        z = rng.standard_normal((B, layers, kv, n, 128))
        chi = (rng.standard_normal((B, layers, kv, n, 128, 4)) ** 2).sum(-1)
        V = (z / np.sqrt(chi / 4)).astype(np.float16)
    else:
        K, V = _kv(rng, B, layers, kv, n, kind)
    s = rng.random((B, n)).astype(np.float32)
    Lh, Ll = (6, 6) if r == 1.0 else (6, 5)
    cache, op = _quantize_case(K, V, s, r, Lh, Ll, f"mfma n={n}")
    for sm in (1.0, 1 / math.sqrt(128)):
        q = (rng.standard_normal((B, layers, Hq, 128)) / math.sqrt(128)).astype(np.float16)
        out = torch.empty((B, layers, Hq, 128), dtype=torch.float32, device="cuda")
        sk.semkv_decode_attn(cache, to_dev(q), out, sm_scale=sm)
        sk.semkv_sync_check()
        assert_attention_close(out.cpu().numpy(), O.decode_attention(q, op, sm),
                               f"mfma n={n} r={r} {kind} sm={sm}")


@pytest.mark.parametrize("L", [3, 4, 5, 6, 8, 16])
def test_decode_mfma_uniform_levels(L):
    _print("decode mfma uniform", L)
    rng = np.random.default_rng(L)
    B, layers, kv, Hq, n = 1, 2, 2, 8, 777
    K, V = _kv(rng, B, layers, kv, n)
    s = rng.random((B, n)).astype(np.float32)
    cache, op = _quantize_case(K, V, s, 0.0, L, L, f"uniform L={L}")
    q = (rng.standard_normal((B, layers, Hq, 128)) / math.sqrt(128)).astype(np.float16)
    out = torch.empty((B, layers, Hq, 128), dtype=torch.float32, device="cuda")
    sk.semkv_decode_attn(cache, to_dev(q), out)
    sk.semkv_sync_check()
    assert_attention_close(out.cpu().numpy(), O.decode_attention(q, op, 1.0), f"uniform {L}")


def test_decode_mfma_large_logits():
    """Peaked softmax: a few tokens dominate, the running maximum moves
    between tiles, and exp() must not overflow."""
    _print("decode mfma peaked")
    rng = np.random.default_rng(99)
    B, layers, kv, Hq, n = 1, 1, 2, 8, 4000
    K, V = _kv(rng, B, layers, kv, n)
    K[:, :, :, 3000:3010] *= 4.0            # late tokens with large keys
    K = K.astype(np.float16)
    s = rng.random((B, n)).astype(np.float32)
    cache, op = _quantize_case(K, V, s, 0.5, 6, 5, "peaked")
    q = rng.standard_normal((B, layers, Hq, 128)).astype(np.float16)      # not pre-scaled
    out = torch.empty((B, layers, Hq, 128), dtype=torch.float32, device="cuda")
    sk.semkv_decode_attn(cache, to_dev(q), out, sm_scale=0.5)
    sk.semkv_sync_check()
    assert_attention_close(out.cpu().numpy(), O.decode_attention(q, op, 0.5), "peaked")


@pytest.mark.parametrize("Lh,Ll", [(5, 4), (6, 4), (6, 6), (5, 5), (16, 16), (16, 6), (16, 5), (16, 4),
                                   (4, 3), (3, 3), (5, 3), (6, 3), (16, 3), (8, 6), (8, 8), (16, 8),
                                   (8, 5), (8, 4), (8, 3)])
@pytest.mark.parametrize("kind", ["normal", "mixed", "studentt"])
def test_decode_mfma_level_pairs(Lh, Ll, kind):
    """Every level pair of the matrix-core kernel, on several tiles with a
    ragged last one, peaked and heavy-tailed values."""
    _print("decode mfma pair", Lh, Ll, kind)
    rng = np.random.default_rng(Lh * 31 + Ll)
    B, layers, kv, Hq, n = 1, 2, 2, 8, 1333
    if kind == "studentt":
        K, _ = _kv(rng, B, layers, kv, n)
        z = rng.standard_normal((B, layers, kv, n, 128))
        chi = (rng.standard_normal((B, layers, kv, n, 128, 4)) ** 2).sum(-1)
        V = (z / np.sqrt(chi / 4)).astype(np.float16)
    else:
        K, V = _kv(rng, B, layers, kv, n, kind)
    s = rng.random((B, n)).astype(np.float32)
    cache, op = _quantize_case(K, V, s, 0.4, Lh, Ll, f"pair ({Lh},{Ll}) {kind}")
    for sm in (1.0, 1 / math.sqrt(128)):
        q = (rng.standard_normal((B, layers, Hq, 128)) / math.sqrt(128)).astype(np.float16)
        out = torch.empty((B, layers, Hq, 128), dtype=torch.float32, device="cuda")
        sk.semkv_decode_attn(cache, to_dev(q), out, sm_scale=sm)
        sk.semkv_sync_check()
        assert_attention_close(out.cpu().numpy(), O.decode_attention(q, op, sm),
                               f"pair ({Lh},{Ll}) {kind} sm={sm}")
