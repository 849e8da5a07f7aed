"""GPU parity of the key-norm score (SemKV Fig. 2 and Table 3; the form read
as the sum of key-row norms over a layer window and the KV heads) against
the oracle, and of the rank taken on it.

Tolerance: each row's sum of 128 squares is exact per product and rounds at
most 34 times in fp32 (32 per lane, 2 across the quad), the square root once,
and the window's nl*kv norms are summed with nl*kv - 1 roundings, so the
relative error is below (nl*kv + 40) * 2^-24 (all terms are non-negative).
The test allows twice that."""
import numpy as np
import pytest
import torch

import oracle as O
from parity_helpers import to_dev

pytestmark = pytest.mark.gpu
sk = pytest.importorskip("kv_cache_mixed_top_amd.semkv")


def _print(*a):
    print(*a, flush=True)


def _tol(nl, kv):
    return (nl * kv + 40) * 2.0 ** -23


def _check(got, ref, nl, kv, what):
    rel = np.abs(got.astype(np.float64) - ref) / np.maximum(ref, 1e-30)
    rel = np.where(ref == 0, np.abs(got), rel)
    assert float(rel.max()) <= _tol(nl, kv), f"{what}: max rel {rel.max():.3e}"


@pytest.mark.parametrize("n", [1, 63, 64, 65, 700])
@pytest.mark.parametrize("window", [(0, 4), (1, 2), (3, 1)])
def test_score_keynorm_small(n, window):
    layer0, nl = window
    _print("score keynorm", n, window)
    rng = np.random.default_rng(n * 7 + layer0)
    B, layers, kv = 2, 4, 3
    K = rng.standard_normal((B, layers, kv, n, 128))
    K[..., 5] *= 10.0                                      # an outlier channel
    if n > 3:
        K[0, :, :, 2, :] = 0.0                             # a zero key everywhere
        K[1, :, :, 3, :] *= 1e-4                           # tiny keys (fp16 subnormals among them)
    K = K.astype(np.float16)
    ld = n + 5
    scores = torch.full((B, ld), -7.0, dtype=torch.float32, device="cuda")
    sk.semkv_score_keynorm(to_dev(K), scores, layer0, nl)
    sk.semkv_sync_check()
    got = scores.cpu().numpy()
    assert np.all(got[:, n:] == -7.0)                      # the row padding is untouched
    _check(got[:, :n], O.score_keynorm(K, layer0, nl), nl, kv, f"n={n} window={window}")


def test_score_keynorm_strided_layout():
    """Tokens outermost ([B][n][layers][kv][128] storage), a token stride of
    layers*kv*128 elements."""
    _print("score keynorm strided")
    rng = np.random.default_rng(5)
    B, layers, kv, n = 2, 3, 2, 333
    store = rng.standard_normal((B, n, layers, kv, 128)).astype(np.float16)
    Kd = to_dev(store).permute(0, 2, 3, 1, 4)              # a view, not a copy
    assert Kd.stride(3) == layers * kv * 128
    scores = torch.empty((B, n), dtype=torch.float32, device="cuda")
    sk.semkv_score_keynorm(Kd, scores, 1, 2)
    sk.semkv_sync_check()
    ref = O.score_keynorm(np.ascontiguousarray(store.transpose(0, 2, 3, 1, 4)), 1, 2)
    _check(scores.cpu().numpy(), ref, 2, kv, "strided")


def test_score_then_rank():
    """The rank of the GPU scores equals the oracle's rank of the same scores
    (bit-exact), and the score order agrees with the oracle's where the
    oracle's scores are apart by more than the tolerance."""
    _print("score then rank")
    rng = np.random.default_rng(9)
    B, layers, kv, n = 2, 4, 8, 4000
    K = (rng.standard_normal((B, layers, kv, n, 128))
         * rng.uniform(0.5, 2.0, (B, 1, 1, n, 1))).astype(np.float16)
    scores = torch.empty((B, n), dtype=torch.float32, device="cuda")
    sk.semkv_score_keynorm(to_dev(K), scores, 0, layers)
    k = O.topr_count(n, 0.5)
    perm = torch.empty((B, n), dtype=torch.int32, device="cuda")
    sk.semkv_rank_topr(scores, k, perm)
    sk.semkv_sync_check()
    s = scores.cpu().numpy()
    wp, _ = O.rank_topr_batch(s, k)
    assert np.array_equal(perm.cpu().numpy(), wp)
    ref = O.score_keynorm(K, 0, layers)
    _check(s, ref, layers, kv, "score then rank")
    hp, _ = O.rank_topr_batch(ref, k)
    for b in range(B):
        got_h, ref_h = set(wp[b, :k]), set(hp[b, :k])
        if got_h != ref_h:                                 # only near-equal scores may swap
            kth = np.sort(ref[b])[::-1][k - 1]
            for t in got_h ^ ref_h:
                assert abs(ref[b, t] - kth) <= 4 * _tol(layers, kv) * kth


def test_score_keynorm_full_size_sampled():
    """llama8b_32k's K (32 layers x 8 KV heads x 32,768 tokens) scored over
    its last 4 layers in the launch bench.py times; 256 sampled tokens
    checked against the oracle on their own rows."""
    _print("score keynorm full size")
    g = torch.Generator(device="cuda").manual_seed(21)
    B, layers, kv, n = 1, 32, 8, 32768
    K = torch.randn((B, layers, kv, n, 128), generator=g, device="cuda").to(torch.float16)
    scores = torch.empty((B, n), dtype=torch.float32, device="cuda")
    sk.semkv_score_keynorm(K, scores, 28, 4)
    sk.semkv_sync_check()
    idx = np.sort(np.random.default_rng(1).choice(n, 256, replace=False))
    rows = K[:, 28:32, :, torch.as_tensor(idx, device="cuda"), :].cpu().numpy()
    ref = O.score_keynorm(rows, 0, 4)
    _check(scores.cpu().numpy()[:, idx], ref, 4, kv, "full size")
    del K


# ---------------------------------------------------------------- hidden-state delta norm
# Tolerance: each update h_j - h_{j-1} is formed in fp32 from two fp16 values
# (relative error <= 2^-24), its square adds one more; lane l sums its
# ceil(d / 512) * 8 squares in order and the wave adds the 64 lane sums in 6
# rounds, so each layer's sum of squares is within (ceil(d/512)*8 + 6 + 3) *
# 2^-24 relative (all terms are non-negative); the square root halves that
# and adds 2^-24, and the S norms are summed with S - 1 roundings.  The test
# allows twice that bound.

def _delta_tol(d, S):
    return 2 * ((-(-d // 512) * 8 + 9) / 2 + 1 + S) * 2.0 ** -24


@pytest.mark.parametrize("d", [64, 1000, 4096])
@pytest.mark.parametrize("states", [2, 5, 9])
def test_score_hidden_delta(d, states):
    _print("score hidden delta", d, states)
    rng = np.random.default_rng(d + states)
    B, n = 2, 300
    h0 = rng.standard_normal((B, 1, n, d))
    steps = rng.standard_normal((B, states - 1, n, d)) * rng.uniform(0.01, 0.5, size=(B, 1, n, 1))
    H = np.concatenate([h0, h0 + np.cumsum(steps, axis=1)], axis=1).astype(np.float16)
    scores = torch.full((B, n + 5), -1.0, dtype=torch.float32, device="cuda")
    sk.semkv_score_hidden_delta(to_dev(H), scores)
    sk.semkv_sync_check()
    got = scores.cpu().numpy()
    ref = O.score_hidden_delta(H)
    rel = np.abs(got[:, :n].astype(np.float64) - ref) / ref
    assert float(rel.max()) <= _delta_tol(d, states - 1), f"max rel {rel.max():.3e}"
    assert np.all(got[:, n:] == -1.0)                         # nothing past n


def test_score_hidden_delta_strided_and_rank():
    """States as a strided view (token-major storage), then the rank of the
    GPU scores equals the oracle's rank of those same scores, bit for bit."""
    _print("score hidden delta strided + rank")
    rng = np.random.default_rng(5)
    B, S1, n, d = 2, 5, 777, 256
    base = rng.standard_normal((B, n, S1, d)).astype(np.float16)     # token-major
    Hv = to_dev(base).permute(0, 2, 1, 3)                           # [B][S1][n][d] view
    scores = torch.empty((B, n), dtype=torch.float32, device="cuda")
    sk.semkv_score_hidden_delta(Hv, scores)
    sk.semkv_sync_check()
    got = scores.cpu().numpy()
    ref = O.score_hidden_delta(np.moveaxis(base, 1, 2))
    rel = np.abs(got.astype(np.float64) - ref) / ref
    assert float(rel.max()) <= _delta_tol(d, S1 - 1)
    k = O.topr_count(n, 0.25)
    perm = torch.empty((B, n), dtype=torch.int32, device="cuda")
    sk.semkv_rank_topr(scores, k, perm)
    sk.semkv_sync_check()
    want, _ = O.rank_topr_batch(got, k)
    assert np.array_equal(perm.cpu().numpy(), want)
