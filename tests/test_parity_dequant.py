"""GPU parity of semkv_dequantize_rows (the reconstruction x = min + code *
scale of the affine quantizer, SemKV Table 6, rotated back by H for a
rotated cache, SemKV Table 2) against the oracle's float64 reconstruction of
the same pool rows.  The kernel computes min + code * scale in fp32, so the
bound is a few fp32 ulps of the row's magnitude (fp32 butterfly sums of 128
terms for rotated rows)."""
import numpy as np
import pytest
import torch

import oracle as O
from parity_helpers import cap16, to_dev

pytestmark = pytest.mark.gpu
sk = pytest.importorskip("kv_cache_mixed_top_amd.semkv")


def _print(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("Lh,Ll,rotate,n,r", [
    (6, 5, False, 700, 0.5), (8, 6, False, 333, 0.25), (16, 4, False, 200, 0.1),
    (65536, 3, False, 150, 0.5), (6, 5, True, 300, 0.5), (5, 4, True, 130, 0.75),
])
def test_dequantize_rows_match_oracle(Lh, Ll, rotate, n, r):
    _print("dequantize", Lh, Ll, rotate, n, r)
    rng = np.random.default_rng(Lh * 7 + Ll + n)
    B, layers, kv = 2, 3, 2
    K = (rng.standard_normal((B, layers, kv, n, 128)) * 2.0).astype(np.float16)
    V = rng.standard_normal((B, layers, kv, n, 128)).astype(np.float16)
    K[..., 3] *= 20.0
    s = rng.random((B, n)).astype(np.float32)
    k = O.topr_count(n, r)
    cache = sk.SemKVCache(B, layers, kv, kv * 4, Lh, Ll, cap16(k), cap16(n - k), rotate=rotate)
    perm = torch.empty((B, n), dtype=torch.int32, device="cuda")
    sk.semkv_rank_topr(to_dev(s), k, perm)
    sk.semkv_quantize_pack(cache, to_dev(K), to_dev(V), perm, k)
    wp, _ = O.rank_topr_batch(s, k)
    op = O.quantize_pack_cache(K, V, wp, k, Lh, Ll, rotate=rotate)
    H = O.hadamard128()
    for high, rows, codes, meta, L in ((True, k, op.codes_high, op.meta_high, Lh),
                                       (False, n - k, op.codes_low, op.meta_low, Ll)):
        if rows == 0:
            continue
        for layer, (r0, nr) in ((0, (0, rows)), (layers - 1, (rows // 3, rows - rows // 3 - 1))):
            if nr <= 0:
                continue
            out = torch.full((B, kv, 2, nr, 128), float("nan"), dtype=torch.float32, device="cuda")
            sk.semkv_dequantize_rows(cache, high, layer, r0, nr, out)
            sk.semkv_sync_check()
            got = out.cpu().numpy().astype(np.float64)
            for b in range(B):
                want = O.dequantize_pool(codes[b, layer], meta[b, layer], L)[:, :, r0:r0 + nr]
                if rotate:
                    want = want @ H                      # rows H x -> x (H symmetric)
                scale = np.maximum(np.abs(want).max(axis=-1, keepdims=True), 1e-30)
                err = float((np.abs(got[b] - want) / scale).max())
                bound = 1e-5 if rotate else 2.0 ** -22   # 128 fp32 adds; one fp32 rounding
                assert err <= bound, f"L={L} high={high} layer={layer} b={b}: {err:.3e}"


def test_dequantize_rejects_bad_ranges():
    cache = sk.SemKVCache(1, 2, 2, 8, 6, 5, 64, 64)
    K = torch.zeros((1, 2, 2, 40, 128), dtype=torch.float16, device="cuda")
    perm = torch.arange(40, dtype=torch.int32, device="cuda")[None].contiguous()
    sk.semkv_quantize_pack(cache, K, K, perm, 20)
    out = torch.zeros((1, 2, 2, 21, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(sk.SemKVError):
        sk.semkv_dequantize_rows(cache, True, 0, 0, 21, out)      # only 20 high rows
    with pytest.raises(sk.SemKVError):
        sk.semkv_dequantize_rows(cache, True, 2, 0, 21, out)      # no layer 2
    sk.semkv_dequantize_rows(cache, False, 1, 0, 20, out[:, :, :, :20].contiguous())
    sk.semkv_sync_check()
