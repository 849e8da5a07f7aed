"""The no-allocation decode entry point (semkv_decode_attn_noalloc): its
partials live in the library's static device scratch.  Its output must match
semkv_decode_attn (the workspace form) and the oracle within the decode
tolerance, on two calls in a row, the second smaller than the first (the
scratch keeps the first call's contents), and a call whose partials exceed
the scratch is refused before anything is launched."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from parity_helpers import TOL, assert_attention_close, cap16, to_dev

pytestmark = pytest.mark.gpu
sk = pytest.importorskip("kv_cache_mixed_top_amd.semkv")


def _print(*a):
    print(*a, flush=True)


def _cache(rng, B, layers, kv, Hq, n, r, Lh, Ll, block=128, gen=0):
    K = rng.standard_normal((B, layers, kv, n, 128)).astype(np.float16)
    V = rng.standard_normal((B, layers, kv, n, 128)).astype(np.float16)
    s = rng.random((B, n)).astype(np.float32)
    k = O.topr_count(n, r)
    tot = n + gen
    cache = sk.SemKVCache(B, layers, kv, Hq, Lh, Ll, cap16(tot), cap16(tot), block=block,
                          max_tokens=tot + block)
    perm = torch.empty((B, n), dtype=torch.int32, device="cuda")
    sk.semkv_rank_topr(to_dev(s), k, perm)
    sk.semkv_quantize_pack(cache, to_dev(K), to_dev(V), perm, k)
    ref = O.GenerationCache(layers=layers, kv_heads=kv, L_high=Lh, L_low=Ll, r=r, block=block,
                            batch=B)
    ref.prompt(K, V, s)
    for _ in range(gen):
        kn = rng.standard_normal((B, layers, kv, 128)).astype(np.float16)
        vn = rng.standard_normal((B, layers, kv, 128)).astype(np.float16)
        sn = rng.random(B).astype(np.float32)
        sk.semkv_append_block(cache, to_dev(kn[:, :, :, None]), to_dev(vn[:, :, :, None]),
                              to_dev(sn[:, None]), r)
        ref.append(kn, vn, sn)
    sk.semkv_sync_check()
    return cache, ref


def _compare(cache, ref, q, layer0, what):
    B, nl, Hq, _ = q.shape
    out_n = torch.full((B, nl, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    out_w = torch.empty_like(out_n)
    sk.semkv_decode_attn_noalloc(cache, to_dev(q), out_n, layer0=layer0)
    sk.semkv_decode_attn(cache, to_dev(q), out_w, layer0=layer0)
    sk.semkv_sync_check()
    a, w = out_n.cpu().numpy(), out_w.cpu().numpy()
    assert np.isfinite(a).all(), what
    d = float((np.abs(a - w) / np.maximum(1.0, np.abs(w))).max())
    assert d <= TOL, f"{what}: no-alloc vs workspace form {d:.3e}"
    e = assert_attention_close(a, ref.decode(q, 1.0, layer0=layer0), what)
    _print(f"{what}: vs workspace form {d:.2e}, vs oracle {e:.2e}")


def test_noalloc_two_calls_second_smaller():
    rng = np.random.default_rng(21)
    # first: the matrix-core path over 3 layers of a 3000-token cache
    c1, r1 = _cache(rng, 2, 3, 2, 8, 3000, 0.5, 6, 5)
    q1 = (rng.standard_normal((2, 3, 8, 128)) / math.sqrt(128)).astype(np.float16)
    _compare(c1, r1, q1, 0, "no-alloc call 1 (3000 tokens, 3 layers)")
    # second, smaller: one layer of a 150-token cache with a generated tail,
    # levels (8, 6) and group 2 (generic kernel); the scratch still holds
    # the first call's partials
    c2, r2 = _cache(rng, 1, 2, 2, 4, 150, 0.25, 8, 6, block=16, gen=21)
    q2 = (rng.standard_normal((1, 1, 4, 128)) / math.sqrt(128)).astype(np.float16)
    _compare(c2, r2, q2, 1, "no-alloc call 2 (171 tokens, 1 layer, tail)")


def test_noalloc_refuses_partials_beyond_the_scratch():
    limit = sk.semkv_decode_noalloc_scratch_bytes()
    assert limit == 64 << 20
    # 160 sequences x 32 layers x 8 KV heads, at least one chunk each: 2080
    # bytes of partials per (sequence, layer, KV head) is above 64 MiB
    B, layers, kv, Hq, n = 160, 32, 8, 32, 16
    assert B * layers * kv * 4 * 130 * 4 > limit
    cache = sk.SemKVCache(B, layers, kv, Hq, 6, 5, 16, 16, block=16, max_decode_layers=1,
                          max_tokens=16)
    K = torch.zeros((B, layers, kv, n, 128), dtype=torch.float16, device="cuda")
    perm = torch.arange(n, dtype=torch.int32, device="cuda").repeat(B, 1).contiguous()
    sk.semkv_quantize_pack(cache, K, K, perm, 8)
    q = torch.zeros((B, layers, Hq, 128), dtype=torch.float16, device="cuda")
    out = torch.zeros((B, layers, Hq, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(sk.SemKVError) as e:
        sk.semkv_decode_attn_noalloc(cache, q, out)
    assert e.value.status == sk.SEMKV_EWORKSPACE
    # one layer of it fits
    sk.semkv_decode_attn_noalloc(cache, q[:, :1].contiguous(), out[:, :1].contiguous())
    sk.semkv_sync_check()
