"""GPU parity at the full workload sizes, on sampled outputs.

The HIP path runs on the whole workload through the same ABI calls the
benchmark times (rank of every sequence, quantize-pack of every layer and KV
head, decode over all layers at once).  The oracle then recomputes, from the
same inputs, what it can in seconds: the complete rank, every row of sampled
(sequence, layer, KV head) planes, and decode outputs of sampled layers or
KV-head groups.  Rows, bytes and meta must be bit-exact; attention within
2e-3 abs/rel.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity_helpers import assert_attention_close, cap16, gpu_plane_rows

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

sk = pytest.importorskip("kv_cache_mixed_top_amd.semkv")
DEV = "cuda"


def _print(*a):
    print(*a, flush=True)


def _inputs(w, seed=0, with_chans=False):
    K, V, chans = W.make_kv_torch(w, DEV, seed=seed)
    if w.score == "attn_mass":
        scores = W.attention_mass_torch(K, w, DEV, seed=seed)
    else:
        g = torch.Generator(device=DEV)
        g.manual_seed(seed + 3)
        scores = torch.rand((w.batch, w.n), generator=g, device=DEV)
    return (K, V, scores, chans) if with_chans else (K, V, scores)


def _rank_full(scores, k):
    B, n = scores.shape
    perm = torch.empty((B, n), dtype=torch.int32, device=DEV)
    mask = torch.empty((B, (n + 31) // 32), dtype=torch.int32, device=DEV)
    sk.semkv_rank_topr(scores, k, perm, mask)
    sk.semkv_sync_check()
    s = scores.cpu().numpy()
    wp, wm = O.rank_topr_batch(s, k)
    assert np.array_equal(perm.cpu().numpy(), wp), "perm differs"
    assert np.array_equal(mask.cpu().numpy().view(np.uint32), wm), "mask differs"
    return perm, wp


def _plane_inputs(K, V, b, layer, head):
    k = K[b, layer, head].cpu().numpy()[None, None, None]
    v = V[b, layer, head].cpu().numpy()[None, None, None]
    return k, v


def _check_plane(cache, K, V, wp, k_high, Lh, Ll, b, layer, head, token_base=0):
    """Every row of one (sequence, layer, KV head) of both pools; returns the
    oracle pools of that plane (kv = 1) for a decode check."""
    kk, vv = _plane_inputs(K, V, b, layer, head)
    op = O.quantize_pack_cache(kk, vv, wp[b:b + 1], k_high, Lh, Ll, token_base=token_base)
    gp = gpu_plane_rows(cache, sk, b, layer, head)
    for name in ("codes_high", "meta_high", "codes_low", "meta_low"):
        a, o = gp[name], getattr(op, name)[0, 0, 0]
        assert a.shape == o.shape, f"{name} ({b},{layer},{head}): {a.shape} != {o.shape}"
        if not np.array_equal(a, o):
            bad = np.argwhere(a != o)
            raise AssertionError(f"{name} ({b},{layer},{head}): {len(bad)} mismatches, "
                                 f"first {bad[:4].tolist()}")
    return op


def _decode_group(op, q, b, layer, head, group, sm, got, what):
    """Decode of the query heads of one KV head against the single-plane oracle pools."""
    qs = q[b, layer, head * group:(head + 1) * group].cpu().numpy()[None, None]
    ref = O.decode_attention(qs, op, sm)[0, 0]
    return assert_attention_close(got[b, layer, head * group:(head + 1) * group], ref, what)


def test_llama8b_32k_full():
    """The benchmark workload: 32 layers x 8 KV heads x 32,768 tokens, r = 0.5."""
    w = W.WORKLOADS["llama8b_32k"]
    _print("llama8b_32k: inputs")
    K, V, scores = _inputs(w)
    n, k = w.n, sk.semkv_topr_count(w.n, w.r)
    perm, wp = _rank_full(scores, k)
    cache = sk.SemKVCache(w.batch, w.layers, w.kv_heads, w.q_heads, 6, 5, cap16(k), cap16(n - k),
                          block=w.block, max_tokens=n)
    sk.semkv_quantize_pack(cache, K, V, perm, k)
    sk.semkv_sync_check()
    assert (cache.n_high, cache.n_low, cache.n_tokens) == (k, n - k, n)
    assert np.array_equal(cache.tok_view(True)[0, :k].cpu().numpy(), wp[0, :k])
    assert np.array_equal(cache.tok_view(False)[0, :n - k].cpu().numpy(), wp[0, k:])
    steps = [0, w.decode_steps - 1]
    q = W.make_q_torch(w, w.decode_steps, DEV)
    outs = []
    for j in range(w.decode_steps):        # the benchmark's decode loop, all layers per launch
        out = torch.empty((w.batch, w.layers, w.q_heads, 128), dtype=torch.float32, device=DEV)
        sk.semkv_decode_partials(cache, q[j], sm_scale=w.sm_scale)
        sk.semkv_decode_merge(cache, out)
        if j in steps:
            outs.append(out)
    # the per-layer launch shape (one layer per partials + merge pair: a few
    # hundred short chunks per head and the many-chunk merge)
    per_layer = {}
    for layer in (0, 31):
        o = torch.empty((w.batch, 1, w.q_heads, 128), dtype=torch.float32, device=DEV)
        sk.semkv_decode_partials(cache, q[0][:, layer:layer + 1].contiguous(), layer0=layer,
                                 sm_scale=w.sm_scale)
        sk.semkv_decode_merge(cache, o)
        per_layer[layer] = o.cpu().numpy()
    sk.semkv_sync_check()
    group = w.q_heads // w.kv_heads
    rng = np.random.default_rng(5)
    extra = [(int(rng.integers(1, 31)), int(rng.integers(0, 8))) for _ in range(4)]
    worst = 0.0
    for layer in (0, 31):
        for head in range(w.kv_heads):
            _print(f"llama8b_32k: plane layer {layer} head {head}")
            op = _check_plane(cache, K, V, wp, k, 6, 5, 0, layer, head)
            for j, out in zip(steps, outs):
                worst = max(worst, _decode_group(op, q[j], 0, layer, head, group, w.sm_scale,
                                                 out.cpu().numpy(), f"step {j} layer {layer}"))
            worst = max(worst, _decode_group(op, q[0][:, layer:layer + 1], 0, 0, head, group,
                                             w.sm_scale, per_layer[layer],
                                             f"per-layer launch, step 0 layer {layer}"))
    # more layers, every KV head: a head's chunks of 4,096 rows each see a
    # different sequence of softmax frames and fixed-point exponents
    for layer in (8, 16, 24):
        for head in range(w.kv_heads):
            extra.append((layer, head))
    for layer, head in extra:
        _print(f"llama8b_32k: plane layer {layer} head {head}")
        op = _check_plane(cache, K, V, wp, k, 6, 5, 0, layer, head)
        for j, out in zip(steps, outs):
            worst = max(worst, _decode_group(op, q[j], 0, layer, head, group, w.sm_scale,
                                             out.cpu().numpy(), f"step {j} layer {layer}"))
    _print(f"llama8b_32k: worst decode error {worst:.3e}")


def test_mix43_r075_sampled():
    """The (4,3) mix at r = 0.75 (SemKV Fig. 18's operating point, affine base)
    at the 8B 32k shape: full rank, sampled planes bit-exact, decode of
    sampled KV-head groups at the first and last of two steps."""
    w = W.WORKLOADS["mix43_r075"]
    _print("mix43_r075: inputs")
    K, V, scores = _inputs(w)
    n, k = w.n, sk.semkv_topr_count(w.n, w.r)
    perm, wp = _rank_full(scores, k)
    cache = sk.SemKVCache(w.batch, w.layers, w.kv_heads, w.q_heads, 4, 3, cap16(k), cap16(n - k),
                          block=w.block, max_tokens=n)
    sk.semkv_quantize_pack(cache, K, V, perm, k)
    q = W.make_q_torch(w, 2, DEV)
    outs = []
    for j in range(2):
        out = torch.empty((w.batch, w.layers, w.q_heads, 128), dtype=torch.float32, device=DEV)
        sk.semkv_decode_attn(cache, q[j], out, sm_scale=w.sm_scale)
        outs.append(out)
    sk.semkv_sync_check()
    for layer, head in ((0, 0), (31, 7), (13, 4)):
        _print(f"mix43_r075: plane layer {layer} head {head}")
        op = _check_plane(cache, K, V, wp, k, 4, 3, 0, layer, head)
        for j in range(2):
            e = _decode_group(op, q[j], 0, layer, head, w.q_heads // w.kv_heads, w.sm_scale,
                              outs[j].cpu().numpy(), f"step {j} layer {layer} head {head}")
            _print(f"   decode error {e:.3e}")


def test_mistral7b_128k_sampled():
    """131,072 tokens, heavy-tailed (Student-t) V, r = 0.5."""
    w = W.WORKLOADS["mistral7b_128k"]
    _print("mistral7b_128k: inputs")
    K, V, scores = _inputs(w)
    n, k = w.n, sk.semkv_topr_count(w.n, w.r)
    perm, wp = _rank_full(scores, k)
    cache = sk.SemKVCache(w.batch, w.layers, w.kv_heads, w.q_heads, 6, 5, cap16(k), cap16(n - k),
                          block=w.block, max_tokens=n)
    sk.semkv_quantize_pack(cache, K, V, perm, k)
    q = W.make_q_torch(w, 1, DEV)[0]
    out = torch.empty((w.batch, w.layers, w.q_heads, 128), dtype=torch.float32, device=DEV)
    sk.semkv_decode_attn(cache, q, out, sm_scale=w.sm_scale)
    sk.semkv_sync_check()
    got = out.cpu().numpy()
    for layer, head in ((31, 3), (0, 6), (17, 0)):
        _print(f"mistral7b_128k: plane layer {layer} head {head}")
        op = _check_plane(cache, K, V, wp, k, 6, 5, 0, layer, head)
        e = _decode_group(op, q, 0, layer, head, w.q_heads // w.kv_heads, w.sm_scale, got,
                          f"layer {layer} head {head}")
        _print(f"   decode error {e:.3e}")


def test_gen_16x8k_sampled():
    """16 x 8,192-token prompts, then 1,024 generated tokens per sequence
    appended one per step and quantized in 128-token blocks."""
    w = W.WORKLOADS["gen_16x8k"]
    _print("gen_16x8k: inputs")
    K, V, scores, chans = _inputs(w, with_chans=True)
    B, n, k = w.batch, w.n, sk.semkv_topr_count(w.n, w.r)
    perm, wp = _rank_full(scores, k)
    T = w.gen_tokens
    kb = sk.semkv_topr_count(w.block, w.r)
    cap_h = cap16(k + (T // w.block + 1) * kb)
    cap_l = cap16(n - k + (T // w.block + 1) * (w.block - kb))
    cache = sk.SemKVCache(B, w.layers, w.kv_heads, w.q_heads, 6, 5, cap_h, cap_l, block=w.block,
                          max_tokens=n + T)
    sk.semkv_quantize_pack(cache, K, V, perm, k)
    # generated tokens with the prompt's distributions (outlier channels too)
    Kg, Vg, Sg = W.make_gen_tokens_torch(w, T, DEV, chans=chans)
    Qg = W.make_q_torch(w, 2, DEV, seed=5)
    layers_s = (0, 31)
    ref = O.GenerationCache(layers=len(layers_s), kv_heads=w.kv_heads, L_high=6, L_low=5,
                            r=w.r, block=w.block, batch=1)
    ref.prompt(K[0:1, list(layers_s)].cpu().numpy(), V[0:1, list(layers_s)].cpu().numpy(),
               scores[0:1].cpu().numpy())
    kg = Kg[:, 0, list(layers_s)].cpu().numpy()
    vg = Vg[:, 0, list(layers_s)].cpu().numpy()
    sg = Sg[:, 0].cpu().numpy()
    check = {w.block - 1: 0, 1000: 1}
    out = torch.empty((B, w.layers, w.q_heads, 128), dtype=torch.float32, device=DEV)
    group = w.q_heads // w.kv_heads
    for i in range(T):
        sk.semkv_append_block(cache, Kg[i].unsqueeze(3), Vg[i].unsqueeze(3), Sg[i].unsqueeze(1),
                              w.r)
        ref.append(kg[i][None], vg[i][None], sg[i:i + 1])
        assert cache.n_tail == ref.n_tail
        if i in check:
            qi = Qg[check[i]]
            sk.semkv_decode_attn(cache, qi, out, sm_scale=w.sm_scale)
            sk.semkv_sync_check()
            qs = qi[0:1, list(layers_s)].cpu().numpy()
            refo = ref.decode(qs, w.sm_scale)
            e = assert_attention_close(out[0:1, list(layers_s)].cpu().numpy(), refo,
                                       f"gen step {i}")
            _print(f"gen_16x8k: step {i}, tail {cache.n_tail}, decode error {e:.3e}")
    sk.semkv_append_block(cache, None, None, None, w.r, flush=True)
    ref.flush()
    sk.semkv_sync_check()
    assert cache.n_high + cache.n_low == n + T and cache.n_tail == 0
    assert cache.n_high == k + (T // w.block) * kb
    for li, layer in enumerate(layers_s):
        for head in range(w.kv_heads):
            gp = gpu_plane_rows(cache, sk, 0, layer, head)
            for name in ("codes_high", "meta_high", "codes_low", "meta_low"):
                assert np.array_equal(gp[name], getattr(ref.pools, name)[0, li, head]), \
                    f"gen {name} layer {layer} head {head}"
    assert np.array_equal(cache.tok_view(True)[0, :cache.n_high].cpu().numpy(),
                          ref.pools.tok_high[0])
    assert np.array_equal(cache.tok_view(False)[0, :cache.n_low].cpu().numpy(),
                          ref.pools.tok_low[0])


def _cliff_settings():
    s = [(L, L, 0.0) for L in W.CLIFF_UNIFORM]
    s += [(Lh, Ll, r) for Lh, Ll in W.CLIFF_PAIRS for r in W.CLIFF_RS]
    return s


def test_cliff_grid_sampled():
    """Batch 4 x 32,768 tokens: every uniform level count and every mixed pair
    x fraction of the sweep, one sampled plane and KV-head group each."""
    w = W.WORKLOADS["cliff_4x32k"]
    _print("cliff_4x32k: inputs")
    K, V, scores = _inputs(w)
    B, n = w.batch, w.n
    q = W.make_q_torch(w, 1, DEV)[0]
    rng = np.random.default_rng(11)
    group = w.q_heads // w.kv_heads
    s_np = scores.cpu().numpy()
    for Lh, Ll, r in _cliff_settings():
        k = sk.semkv_topr_count(n, r)
        perm = torch.empty((B, n), dtype=torch.int32, device=DEV)
        sk.semkv_rank_topr(scores, k, perm)
        cache = sk.SemKVCache(B, w.layers, w.kv_heads, w.q_heads, Lh, Ll, cap16(k),
                              cap16(n - k), block=w.block, max_tokens=n)
        sk.semkv_quantize_pack(cache, K, V, perm, k)
        out = torch.empty((B, w.layers, w.q_heads, 128), dtype=torch.float32, device=DEV)
        sk.semkv_decode_attn(cache, q, out, sm_scale=w.sm_scale)
        sk.semkv_sync_check()
        wp, _ = O.rank_topr_batch(s_np, k)
        assert np.array_equal(perm.cpu().numpy(), wp)
        b, layer, head = int(rng.integers(0, B)), int(rng.integers(0, 32)), int(rng.integers(0, 8))
        op = _check_plane(cache, K, V, wp, k, Lh, Ll, b, layer, head)
        e = _decode_group(op, q, b, layer, head, group, w.sm_scale, out.cpu().numpy(),
                          f"cliff ({Lh},{Ll}) r={r}")
        _print(f"cliff ({Lh},{Ll}) r={r}: plane ({b},{layer},{head}) exact, decode error {e:.3e}")
        del cache, out
        torch.cuda.empty_cache()


def _frame_raise_case(n, layers_checked, heads_checked, bound, what):
    """Logits shaped so that every chunk of a 32-layer launch first lowers
    its fixed-point exponent (a few tokens just under the softmax frame) and
    then raises its frame (a spike 11.5 nats above the typical tokens, whose
    weights after the raise are small); the pattern repeats every 2,048
    rows.  The decode error against the oracle is held to `bound`."""
    B, layers, kv, Hq, r = 1, 32, 8, 32, 0.5
    beta = 10.0 / 3.0                                   # logit per unit of the u component
    g = torch.Generator(device=DEV)
    g.manual_seed(21)
    u = torch.randn((layers, kv, 128), generator=g, device=DEV)
    u = u / u.norm(dim=-1, keepdim=True)
    a = 0.3 * torch.randn((n,), generator=g, device=DEV)           # typical logits ~ N(0, 1)
    pos = torch.arange(n, device=DEV) % 2048
    for off in (200, 260, 320, 380):
        a = torch.where(pos == off, torch.full_like(a, 3.0), a)     # just under the frame: 10 nats
    for off in (1100, 1160):
        a = torch.where(pos == off, torch.full_like(a, 3.45), a)    # the spike: 11.5 nats
    K = (0.05 * torch.randn((B, layers, kv, n, 128), generator=g, device=DEV)
         + a[None, None, None, :, None] * u[None, :, :, None, :]).half()
    V = torch.randn((B, layers, kv, n, 128), generator=g, device=DEV).half()
    q = (beta * u.repeat_interleave(Hq // kv, dim=1)[None]
         + 0.02 * torch.randn((B, layers, Hq, 128), generator=g, device=DEV)).half()
    scores = torch.rand((B, n), generator=g, device=DEV)
    k = sk.semkv_topr_count(n, r)
    perm, wp = _rank_full(scores, k)
    cache = sk.SemKVCache(B, layers, kv, Hq, 6, 5, cap16(k), cap16(n - k), max_tokens=n)
    sk.semkv_quantize_pack(cache, K, V, perm, k)
    out = torch.empty((B, layers, Hq, 128), dtype=torch.float32, device=DEV)
    sk.semkv_decode_partials(cache, q)
    sk.semkv_decode_merge(cache, out)
    sk.semkv_sync_check()
    got = out.cpu().numpy()
    worst = 0.0
    for layer in layers_checked:
        for head in heads_checked:
            op = _check_plane(cache, K, V, wp, k, 6, 5, 0, layer, head)
            worst = max(worst, _decode_group(op, q, 0, layer, head, Hq // kv, 1.0, got,
                                             f"{what} layer {layer} head {head}"))
    _print(f"{what}: worst decode error {worst:.3e}")
    assert worst <= bound, f"{what}: {worst:.3e} > {bound:.1e}"


def test_decode_frame_raise_after_lowered_exponent():
    """8,192 tokens: the launch takes 1,024-row chunks.  Besides the 2e-3
    parity bound the error is held to 2e-5, ten times what the arithmetic
    allows: the weights keep at least 28 bits against a chunk's largest
    weight (an error below rows / 2^29 = 1.9e-6 of its normaliser) and the
    query 27 bits, so a larger error means lost weight bits.  (An exponent
    kept across the frame raise leaves the typical tokens' weights at a few
    units: 1.6e-4 here.)"""
    _frame_raise_case(8192, (0, 17), range(8), 2e-5, "frame raise, 1,024-row chunks")


def test_decode_frame_raise_long_chunks():
    """65,536 tokens: the launch fits one round of 8,192-row chunks (the
    single-round rule; the kernel takes chunks up to 16,384 rows).  The bound
    is ten times the weights' error for the longest such chunk,
    10 x 16,384 / 2^29 = 3.1e-4 of a chunk's normaliser."""
    _frame_raise_case(65536, (5,), (0, 7), 3.1e-4, "frame raise, long chunks")
