"""Helpers shared by the GPU parity tests (marshalling and comparison only)."""
import numpy as np
import torch

import oracle as O

TOL = 2e-3   # decode attention: |gpu - oracle| <= TOL * max(1, |oracle|)


def cap16(x):
    return max(16, (int(x) + 15) // 16 * 16)


def assert_attention_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref) / np.maximum(1.0, np.abs(ref))
    worst = float(err.max()) if err.size else 0.0
    assert worst <= TOL, f"{what}: max abs/rel error {worst:.3e} > {TOL}"
    return worst


def planar_rows(plane, R, n):
    """Rows 0..n-1 of a byte-planar plane (byte j of row r at
    (r // 16) * 16 * R + 16 * j + r % 16) as [..., n, R]."""
    r = np.arange(n)[:, None]
    j = np.arange(R)[None, :]
    return plane[..., (r // 16) * 16 * R + 16 * j + (r % 16)]


def gpu_pools(cache, sk):
    """Valid rows of the device pools as numpy arrays in the oracle's layout.

    K planes hold rows back to back; V planes are byte-planar in 16-row
    tiles (include/semkv.h)."""
    g = cache.geom
    out = {}
    for name, high, n in (("high", True, cache.n_high), ("low", False, cache.n_low)):
        L = g.L_high if high else g.L_low
        cap = g.cap_high if high else g.cap_low
        R = sk.semkv_row_bytes(L)
        raw = (cache.codes_high if high else cache.codes_low).view(
            g.batch, g.layers, g.kv_heads, 2, cap * R).cpu().numpy()
        k_rows = raw[..., 0, :n * R].reshape(g.batch, g.layers, g.kv_heads, n, R)
        v_rows = planar_rows(raw[..., 1, :], R, n)
        out["codes_" + name] = np.stack([k_rows, v_rows], axis=3)
        out["meta_" + name] = cache.meta_view(high)[..., :n, :].cpu().numpy().view(np.uint16)
        out["tok_" + name] = cache.tok_view(high)[:, :n].cpu().numpy()
    return out


def assert_pools_equal(gp, op: "O.Pools", what=""):
    for name in ("codes_high", "codes_low", "meta_high", "meta_low", "tok_high", "tok_low"):
        a = gp[name]
        b = getattr(op, name)
        assert a.shape == b.shape, f"{what} {name}: shape {a.shape} != {b.shape}"
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)
            raise AssertionError(f"{what} {name}: {len(bad)} mismatches, first at {bad[:5].tolist()}")


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def gpu_plane_rows(cache, sk, b, layer, head):
    """Valid rows of one (sequence, layer, KV head) of both device pools:
    {"codes_high": [2][n_high][R], "meta_high": [2][n_high][2], ...} with
    index 0 = K, 1 = V (V un-transposed from its byte-planar tiles)."""
    g = cache.geom
    out = {}
    for name, high, n in (("high", True, cache.n_high), ("low", False, cache.n_low)):
        L = g.L_high if high else g.L_low
        cap = g.cap_high if high else g.cap_low
        R = sk.semkv_row_bytes(L)
        codes = (cache.codes_high if high else cache.codes_low).view(
            g.batch, g.layers, g.kv_heads, 2, cap * R)[b, layer, head].cpu().numpy()
        k_rows = codes[0, :n * R].reshape(n, R)
        v_rows = planar_rows(codes[1], R, n)
        out["codes_" + name] = np.stack([k_rows, v_rows])
        out["meta_" + name] = cache.meta_view(high)[b, layer, head, :, :n, :].cpu().numpy().view(
            np.uint16)
    return out
