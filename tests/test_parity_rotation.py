"""GPU parity of the optional Hadamard rotation (SemKV Table 2's quantizer
with its rotation; the matrix and precision as read in the oracle):
rotated quantize-pack bit-exact against the oracle, decode over rotated pools
within the decode tolerance, and the unsupported combinations refused."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from parity_helpers import assert_attention_close, assert_pools_equal, cap16, gpu_pools, to_dev

pytestmark = pytest.mark.gpu
sk = pytest.importorskip("kv_cache_mixed_top_amd.semkv")


def _print(*a):
    print(*a, flush=True)


def _rows(rng, B, layers, kv, n, kind):
    shape = (B, layers, kv, n, 128)
    K = rng.standard_normal(shape)
    V = rng.standard_normal(shape)
    if kind == "outlier":
        K[..., 3] *= 30.0                                 # one large K channel
        K[..., 77] *= -12.0
    elif kind == "mixed":
        K[..., 5, :] = 1.5                                # a constant row (its rotation is e0-like)
        K[..., 6, :] = 0.0                                # a zero row
        V[..., 2, :] *= 1e-3
        V[..., 9, 40] = 300.0
        # rows along e0 rotate to (nearly) constant rows: a range of a few
        # fp32 ulps above the fp16 floor of the minimum, so |m|/s is large
        for j, (c, dl) in enumerate([(181.0, 0.0), (1000.0, 2.0 ** -13), (3.0, 2.0 ** -20),
                                     (-77.5, 2.0 ** -16)]):
            K[..., 10 + j, :] = 0.0
            K[..., 10 + j, 0] = c
            K[..., 10 + j, 1 + j] = dl
            V[..., 10 + j, :] = 0.0
            V[..., 10 + j, 0] = -c
            V[..., 10 + j, 64] = dl
    return K.astype(np.float16), V.astype(np.float16)


def _rotated_case(K, V, scores, r, what):
    B, layers, kv, n, _ = K.shape
    k = O.topr_count(n, r)
    cache = sk.SemKVCache(B, layers, kv, kv * 4, 6, 5, cap16(k), cap16(n - k), block=128,
                          rotate=True)
    perm = torch.empty((B, n), dtype=torch.int32, device="cuda")
    sk.semkv_rank_topr(to_dev(scores), k, perm)
    sk.semkv_quantize_pack(cache, to_dev(K), to_dev(V), perm, k)
    sk.semkv_sync_check()
    wp, _ = O.rank_topr_batch(scores, k)
    assert np.array_equal(perm.cpu().numpy(), wp), what
    op = O.quantize_pack_cache(K, V, wp, k, 6, 5, rotate=True)
    assert_pools_equal(gpu_pools(cache, sk), op, what)
    return cache, op


@pytest.mark.parametrize("n,r,kind", [(1, 0.5, "normal"), (203, 0.5, "outlier"),
                                      (130, 0.25, "mixed"), (700, 0.75, "normal")])
def test_rotated_quantize_bit_exact(n, r, kind):
    _print("rotated quantize", n, r, kind)
    rng = np.random.default_rng(n + int(10 * r))
    K, V = _rows(rng, 2, 2, 2, n, kind)
    s = rng.random((2, n)).astype(np.float32)
    _rotated_case(K, V, s, r, f"rotated quantize n={n} {kind}")


@pytest.mark.parametrize("n,r,kind,sm", [(63, 0.5, "normal", 1.0), (700, 0.5, "outlier", 1.0),
                                         (3000, 0.25, "mixed", 1 / math.sqrt(128)),
                                         (10000, 0.5, "normal", 1.0)])
def test_rotated_decode(n, r, kind, sm):
    _print("rotated decode", n, r, kind)
    rng = np.random.default_rng(3 * n + 1)
    B, layers, kv, Hq = 1, 2, 2, 8
    K, V = _rows(rng, B, layers, kv, n, kind)
    s = rng.random((B, n)).astype(np.float32)
    cache, op = _rotated_case(K, V, s, r, f"rotated decode setup n={n}")
    q = (rng.standard_normal((B, layers, Hq, 128)) / math.sqrt(128)).astype(np.float16)
    ref = O.decode_attention(q, op, sm)
    out = torch.empty((B, layers, Hq, 128), dtype=torch.float32, device="cuda")
    sk.semkv_decode_attn(cache, to_dev(q), out, sm_scale=sm)
    sk.semkv_sync_check()
    assert_attention_close(out.cpu().numpy(), ref, f"rotated decode n={n}")
    # per-layer launches (few units: short chunks and the per-query-head merge)
    out_l = torch.empty_like(out)
    for layer in range(layers):
        sk.semkv_decode_partials(cache, to_dev(q[:, layer:layer + 1]), layer0=layer, sm_scale=sm)
        sk.semkv_decode_merge(cache, out_l[:, layer:layer + 1])
    sk.semkv_sync_check()
    assert_attention_close(out_l.cpu().numpy(), ref, f"rotated per-layer decode n={n}")


@pytest.mark.parametrize("Lh,Ll,Hq,n,r,kind", [
    (5, 4, 8, 700, 0.5, "outlier"),         # 5/4 pair, group 4: generic decode
    (8, 6, 8, 333, 0.25, "mixed"),          # 8/6 pair
    (6, 5, 2, 500, 0.5, "outlier"),         # group 1
    (6, 5, 4, 257, 0.75, "mixed"),          # group 2
    (6, 5, 16, 300, 0.5, "normal"),         # group 8
    (16, 4, 8, 200, 0.1, "outlier"),
    (65536, 65536, 8, 90, 0.5, "normal"),
])
def test_rotated_any_levels_and_groups(Lh, Ll, Hq, n, r, kind):
    """Rotation on every level pair and query group: the rotated quantizer
    (generic tile) bit-exact, decode over the generic kernel within the
    tolerance (one launch, and per layer)."""
    _print("rotated any", Lh, Ll, Hq, n, r, kind)
    rng = np.random.default_rng(Lh + Ll + Hq + n)
    B, layers, kv = 2, 2, 2
    K, V = _rows(rng, B, layers, kv, n, kind)
    s = rng.random((B, n)).astype(np.float32)
    k = O.topr_count(n, r)
    cache = sk.SemKVCache(B, layers, kv, Hq, Lh, Ll, cap16(k), cap16(n - k), rotate=True)
    perm = torch.empty((B, n), dtype=torch.int32, device="cuda")
    sk.semkv_rank_topr(to_dev(s), k, perm)
    sk.semkv_quantize_pack(cache, to_dev(K), to_dev(V), perm, k)
    sk.semkv_sync_check()
    wp, _ = O.rank_topr_batch(s, k)
    op = O.quantize_pack_cache(K, V, wp, k, Lh, Ll, rotate=True)
    assert_pools_equal(gpu_pools(cache, sk), op, f"rotated ({Lh},{Ll}) Hq={Hq}")
    q = (rng.standard_normal((B, layers, Hq, 128)) / math.sqrt(128)).astype(np.float16)
    ref = O.decode_attention(q, op, 1.0)
    out = torch.empty((B, layers, Hq, 128), dtype=torch.float32, device="cuda")
    sk.semkv_decode_attn(cache, to_dev(q), out)
    sk.semkv_sync_check()
    e = assert_attention_close(out.cpu().numpy(), ref, f"rotated ({Lh},{Ll}) Hq={Hq} decode")
    for layer in range(layers):
        o1 = torch.empty((B, 1, Hq, 128), dtype=torch.float32, device="cuda")
        sk.semkv_decode_attn(cache, to_dev(q[:, layer:layer + 1]), o1, layer0=layer)
        sk.semkv_sync_check()
        assert_attention_close(o1.cpu().numpy(), ref[:, layer:layer + 1],
                               f"rotated ({Lh},{Ll}) Hq={Hq} layer {layer}")
    _print(f"   decode error {e:.3e}")


@pytest.mark.parametrize("block,n0,steps,r,Lh,Ll,Hq", [
    (128, 150, 300, 0.25, 6, 5, 8), (16, 70, 53, 0.35, 6, 5, 8), (512, 200, 130, 0.5, 6, 5, 8),
    (64, 50, 100, 0.5, 6, 6, 8),            # uniform levels, matrix-core decode
    (16, 40, 45, 0.25, 8, 6, 4),            # generic decode with a tail, group 2
    (32, 33, 70, 0.5, 5, 4, 16),            # group 8
])
def test_rotated_generation(block, n0, steps, r, Lh, Ll, Hq):
    """Generation on a rotated cache (SemKV Fig. 6 with Table 2's rotated
    quantizer): full blocks are rotated and quantized, the fp16 tail is read
    unrotated; pools bit-exact and decode (one launch and per layer) within
    the decode tolerance at steps inside and at the ends of blocks."""
    _print("rotated generation", block, n0, steps, r, Lh, Ll, Hq)
    rng = np.random.default_rng(block + steps)
    B, layers, kv = 2, 2, 2
    K0, V0 = _rows(rng, B, layers, kv, n0, "outlier")
    s0 = rng.random((B, n0)).astype(np.float32)
    k0 = O.topr_count(n0, r)
    tot = n0 + steps
    cache = sk.SemKVCache(B, layers, kv, Hq, Lh, Ll, cap16(tot), cap16(tot), block=block,
                          max_tokens=tot + block, rotate=True)
    perm = torch.empty((B, n0), dtype=torch.int32, device="cuda")
    sk.semkv_rank_topr(to_dev(s0), k0, perm)
    sk.semkv_quantize_pack(cache, to_dev(K0), to_dev(V0), perm, k0)
    ref = O.GenerationCache(layers=layers, kv_heads=kv, L_high=Lh, L_low=Ll, r=r, block=block,
                            batch=B, rotate=True)
    ref.prompt(K0, V0, s0)
    ks = rng.standard_normal((steps, B, layers, kv, 128)).astype(np.float16)
    vs = rng.standard_normal((steps, B, layers, kv, 128)).astype(np.float16)
    ss = rng.random((steps, B)).astype(np.float32)
    out = torch.empty((B, layers, Hq, 128), dtype=torch.float32, device="cuda")
    check_at = {0, block - 1, block, steps - 1}
    for i in range(steps):
        sk.semkv_append_block(cache, to_dev(ks[i][:, :, :, None, :]), to_dev(vs[i][:, :, :, None, :]),
                              to_dev(ss[i][:, None]), r)
        ref.append(ks[i], vs[i], ss[i])
        assert cache.n_tail == ref.n_tail
        if i in check_at:
            q = (rng.standard_normal((B, layers, Hq, 128)) / math.sqrt(128)).astype(np.float16)
            want = ref.decode(q, 1.0)
            sk.semkv_decode_attn(cache, to_dev(q), out)
            sk.semkv_sync_check()
            assert_attention_close(out.cpu().numpy(), want, f"rotated gen step {i}")
            for layer in range(layers):
                o1 = torch.empty((B, 1, Hq, 128), dtype=torch.float32, device="cuda")
                sk.semkv_decode_partials(cache, to_dev(q[:, layer:layer + 1]), layer0=layer)
                sk.semkv_decode_merge(cache, o1)
                sk.semkv_sync_check()
                assert_attention_close(o1.cpu().numpy(), want[:, layer:layer + 1],
                                       f"rotated gen step {i} layer {layer}")
    sk.semkv_append_block(cache, None, None, None, r, flush=True)
    ref.flush()
    sk.semkv_sync_check()
    assert cache.n_tail == 0
    assert_pools_equal(gpu_pools(cache, sk), ref.pools, "rotated generation after flush")


@pytest.mark.parametrize("Lh,Ll,kind", [(6, 6, "outlier"), (5, 5, "outlier"), (6, 6, "mixed"),
                                         (5, 5, "mixed")])
def test_rotated_uniform_levels(Lh, Ll, kind):
    """Rotation on caches of one level count (the generic quantize tile with
    the rotation, the matrix-core decode): bit-exact pools, decode within
    the tolerance."""
    _print("rotated uniform", Lh, Ll, kind)
    rng = np.random.default_rng(Lh * 10 + Ll)
    B, layers, kv, Hq, n = 1, 2, 2, 8, 900
    K, V = _rows(rng, B, layers, kv, n, kind)
    s = rng.random((B, n)).astype(np.float32)
    k = O.topr_count(n, 0.5)
    cache = sk.SemKVCache(B, layers, kv, Hq, Lh, Ll, cap16(k), cap16(n - k), rotate=True)
    perm = torch.empty((B, n), dtype=torch.int32, device="cuda")
    sk.semkv_rank_topr(to_dev(s), k, perm)
    sk.semkv_quantize_pack(cache, to_dev(K), to_dev(V), perm, k)
    sk.semkv_sync_check()
    wp, _ = O.rank_topr_batch(s, k)
    op = O.quantize_pack_cache(K, V, wp, k, Lh, Ll, rotate=True)
    assert_pools_equal(gpu_pools(cache, sk), op, f"rotated ({Lh},{Ll})")
    q = (rng.standard_normal((B, layers, Hq, 128)) / math.sqrt(128)).astype(np.float16)
    out = torch.empty((B, layers, Hq, 128), dtype=torch.float32, device="cuda")
    sk.semkv_decode_attn(cache, to_dev(q), out)
    sk.semkv_sync_check()
    assert_attention_close(out.cpu().numpy(), O.decode_attention(q, op, 1.0), f"rotated ({Lh},{Ll}) decode")

