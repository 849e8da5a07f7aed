"""GPU parity of ragged batches (SemKV Fig. 6 per prompt and per block;
Table 2, multi-turn) against the per-sequence oracle: sequences with their
own prompt lengths, generation pace, end-of-turn flushes and a second turn
share one cache, with every counter on the device.  Pools, tails and
counters must match bit for bit; decode within the attention tolerance."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from kv_cache_mixed_top_amd import semkv as sk
from parity_helpers import assert_attention_close, cap16, planar_rows, to_dev

pytestmark = pytest.mark.gpu


def _print(*a):
    print("[ragged]", *a, flush=True)


def _seq_pools(cache, b, nh, nl):
    """Sequence b's valid pool rows in the oracle's layout (batch axis 1)."""
    g = cache.geom
    out = {}
    for name, high, n in (("high", True, nh), ("low", False, nl)):
        L = g.L_high if high else g.L_low
        cap = g.cap_high if high else g.cap_low
        R = sk.semkv_row_bytes(L)
        raw = (cache.codes_high if high else cache.codes_low).view(
            g.batch, g.layers, g.kv_heads, 2, cap * R)[b].cpu().numpy()
        k_rows = raw[..., 0, :n * R].reshape(g.layers, g.kv_heads, n, R)
        v_rows = planar_rows(raw[..., 1, :], R, n)
        out["codes_" + name] = np.stack([k_rows, v_rows], axis=2)
        out["meta_" + name] = cache.meta_view(high)[b, :, :, :, :n].cpu().numpy().view(np.uint16)
        out["tok_" + name] = cache.tok_view(high)[b, :n].cpu().numpy()
    return out


def _check_state(cache, seq, R, what):
    counts = seq.cpu().numpy()
    g = cache.geom
    for b in range(g.batch):
        nh, nl, nt, ntok = R.counters(b)
        assert tuple(counts[b, :4]) == (nh, nl, nt, ntok), f"{what}: counters of sequence {b}"
        assert counts[b, sk.SEQ_STATUS] == 0, f"{what}: status of sequence {b}"
        gp = _seq_pools(cache, b, nh, nl)
        op = R.pools(b)
        for f in ("codes_high", "codes_low", "meta_high", "meta_low", "tok_high", "tok_low"):
            want = getattr(op, f)[0]
            assert np.array_equal(gp[f], want), f"{what}: {f} of sequence {b}"
        tail = cache.tail_view()[b, :, :, :, :nt].cpu().numpy()
        assert np.array_equal(tail, R.tail_array(b)[:, :, :, :nt]), f"{what}: tail of sequence {b}"


def _check_decode(cache, seq, R, rng, bounds, sm, what):
    g = cache.geom
    q = (rng.standard_normal((g.batch, g.layers, g.q_heads, 128)) / math.sqrt(128)).astype(np.float16)
    out = torch.empty((g.batch, g.layers, g.q_heads, 128), dtype=torch.float32, device="cuda")
    sk.semkv_ragged_decode_attn(cache, seq, to_dev(q), out, bounds[0], bounds[1], sm_scale=sm)
    sk.semkv_sync_check()
    got = out.cpu().numpy()
    for b in range(g.batch):
        assert_attention_close(got[b], R.decode(b, q[b], sm), f"{what}: decode of sequence {b}")


@pytest.mark.parametrize("Hq,rotate,levels", [(8, False, (6, 5)), (4, False, (6, 5)), (8, True, (6, 5)),
                                              (8, False, (5, 4))])
def test_ragged_generation(Hq, rotate, levels):
    """Three sequences: prompts of 150, 300 and 77 tokens; sequence 0 generates
    every step, 1 every other step, 2 ends its turn at step 40 and starts a
    second turn (a 45-token prompt) at step 50; 1 and 0 flush late."""
    _print("generation Hq", Hq, "rotate", rotate, "levels", levels)
    rng = np.random.default_rng(Hq + 10 * rotate + levels[1])
    B, layers, kv, r, block = 3, 2, 2, 0.35, 32
    Lh, Ll = levels
    n_seq = [150, 300, 77]
    n_max = max(n_seq)
    cache = sk.SemKVCache(B, layers, kv, Hq, Lh, Ll, cap16(256), cap16(448), block=block, rotate=rotate)
    seq = torch.zeros((B, sk.SEQ_WORDS), dtype=torch.int64, device="cuda")
    sk.semkv_seq_reset(seq)
    R = O.RaggedGeneration(B, layers, kv, Lh, Ll, r=r, block=block, rotate=rotate)

    def prompt(ns):
        nm = max(ns)
        K = rng.standard_normal((B, layers, kv, nm, 128)).astype(np.float16)
        V = rng.standard_normal((B, layers, kv, nm, 128)).astype(np.float16)
        s = rng.random((B, nm)).astype(np.float32)
        for b in range(B):
            s[b, ns[b]:] = 10.0           # past a sequence's prompt: larger than any real score
        perm = torch.empty((B, nm), dtype=torch.int32, device="cuda")
        nd = to_dev(np.asarray(ns, np.int32))
        sk.semkv_ragged_rank_topr(to_dev(s), nd, r, perm)
        sk.semkv_ragged_quantize_pack(cache, seq, to_dev(K), to_dev(V), nd, r, perm)
        for b in range(B):
            if ns[b] > 0:
                R.prompt(b, K[b, :, :, :ns[b]], V[b, :, :, :ns[b]], s[b, :ns[b]])

    prompt(n_seq)
    sk.semkv_sync_check()
    _check_state(cache, seq, R, "after prompts")
    _check_decode(cache, seq, R, rng, (cache.geom.cap_high, cache.geom.cap_low), 1.0, "after prompts")

    for step in range(90):
        if step == 50:
            prompt([0, 0, 45])                                         # second turn of sequence 2
            continue
        active = np.array([1, step % 2 == 0, step < 40 or step > 50], np.int32)
        flush = np.array([step == 85, step == 70, step == 40], np.int32)
        kn = rng.standard_normal((B, layers, kv, 1, 128)).astype(np.float16)
        vn = rng.standard_normal((B, layers, kv, 1, 128)).astype(np.float16)
        sc = rng.random(B).astype(np.float32)
        sk.semkv_ragged_append(cache, seq, to_dev(kn), to_dev(vn), to_dev(sc), to_dev(active), r,
                               flush=to_dev(flush))
        for b in range(B):
            if active[b]:
                R.append(b, kn[b, :, :, 0], vn[b, :, :, 0], sc[b])
            if flush[b]:
                R.flush(b)
        if step in (30, 45, 89):   # step 30: tails of 31 (block - 1), 16 and 31 rows
            sk.semkv_sync_check()
            _check_state(cache, seq, R, f"step {step}")
            nh = max(R.counters(b)[0] for b in range(B))
            nl = max(R.counters(b)[1] for b in range(B))
            _check_decode(cache, seq, R, rng, (nh, nl), 1 / math.sqrt(128), f"step {step}")


def test_ragged_capacity_and_busy_tail_status():
    """A prompt that does not fit, and a prompt while the tail holds tokens,
    write nothing for that sequence, set its status bit and leave its
    counters; the other sequences go on as usual."""
    _print("capacity / busy tail")
    rng = np.random.default_rng(7)
    B, layers, kv, Hq, r = 2, 1, 2, 8, 0.5
    cache = sk.SemKVCache(B, layers, kv, Hq, 6, 5, 32, 64, block=16)
    seq = torch.zeros((B, sk.SEQ_WORDS), dtype=torch.int64, device="cuda")
    sk.semkv_seq_reset(seq)
    R = O.RaggedGeneration(B, layers, kv, 6, 5, r=r, block=16)
    ns = [40, 100]                       # 100 tokens need 50 high rows > 32
    K = rng.standard_normal((B, layers, kv, 100, 128)).astype(np.float16)
    V = rng.standard_normal((B, layers, kv, 100, 128)).astype(np.float16)
    s = rng.random((B, 100)).astype(np.float32)
    perm = torch.empty((B, 100), dtype=torch.int32, device="cuda")
    nd = to_dev(np.asarray(ns, np.int32))
    sk.semkv_ragged_rank_topr(to_dev(s), nd, r, perm)
    sk.semkv_ragged_quantize_pack(cache, seq, to_dev(K), to_dev(V), nd, r, perm)
    R.prompt(0, K[0, :, :, :40], V[0, :, :, :40], s[0, :40])
    sk.semkv_sync_check()
    counts = seq.cpu().numpy()
    assert tuple(counts[0, :5]) == R.counters(0) + (0,)
    assert tuple(counts[1, :4]) == (0, 0, 0, 0) and counts[1, sk.SEQ_STATUS] == 1   # capacity
    gp = _seq_pools(cache, 0, 20, 20)
    assert np.array_equal(gp["codes_high"], R.pools(0).codes_high[0])
    # one token into sequence 0's tail, then a prompt for it: skipped (busy)
    kn = rng.standard_normal((B, layers, kv, 1, 128)).astype(np.float16)
    sk.semkv_ragged_append(cache, seq, to_dev(kn), to_dev(kn), to_dev(np.ones(B, np.float32)),
                           to_dev(np.array([1, 0], np.int32)), r)
    nd2 = to_dev(np.array([10, 0], np.int32))
    perm2 = torch.empty((B, 10), dtype=torch.int32, device="cuda")
    sk.semkv_ragged_rank_topr(to_dev(s[:, :10].copy()), nd2, r, perm2)
    sk.semkv_ragged_quantize_pack(cache, seq, to_dev(K[:, :, :, :10].copy()), to_dev(V[:, :, :, :10].copy()),
                                  nd2, r, perm2)
    sk.semkv_sync_check()
    counts = seq.cpu().numpy()
    assert tuple(counts[0, :4]) == (20, 20, 1, 41) and counts[0, sk.SEQ_STATUS] == 2
