"""Host side of the C ABI: the library loads, exports every function that
include/semkv.h declares, answers the size queries, and rejects invalid
arguments with the documented status before anything is launched.  No call
here reaches the GPU."""
import ctypes
import os
import re

import pytest

import oracle as O
from conftest import ROOT

sk = pytest.importorskip("kv_cache_mixed_top_amd.semkv",
                         reason="libsemkv.so not built (python -m kv_cache_mixed_top_amd.build)")


def header_functions():
    text = open(os.path.join(ROOT, "include", "semkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(semkv_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 12
    lib = ctypes.CDLL(sk.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(sk.EXPORTED)


def test_row_bytes_match_oracle_layout():
    for L in [3, 4, 5, 6, 7, 8, 9, 16, 100, 255, 256, 257, 1000, 65535, 65536]:
        assert sk.semkv_row_bytes(L) == O.row_bytes(L)
    assert sk.semkv_row_bytes(2) < 0 and sk.semkv_row_bytes(65537) < 0


def test_topr_count_matches_oracle():
    for n in [0, 1, 2, 7, 128, 512, 8192, 32768, 131072]:
        for r in [0.0, 0.1, 0.25, 0.35, 0.5, 0.75, 0.9, 1.0]:
            assert sk.semkv_topr_count(n, r) == O.topr_count(n, r)
    assert sk.semkv_topr_count(10, 1.5) < 0 and sk.semkv_topr_count(-1, 0.5) < 0


def geom(**kw):
    d = dict(batch=1, layers=32, kv_heads=8, q_heads=32, head_dim=128, L_high=6, L_low=5,
             block=128, cap_high=16384, cap_low=16384)
    d.update(kw)
    return sk.semkv_geom(**d)


def test_rotated_geometry_accepted():
    """Rotation is a quantizer option for every level pair and query group."""
    out = (ctypes.c_int64 * 8)()
    assert sk._lib.semkv_cache_sizes(ctypes.byref(geom(rotate=1)), out) == sk.SEMKV_OK
    for lh, ll, hq in ((6, 6, 32), (5, 5, 32), (8, 6, 32), (6, 4, 32), (16, 3, 32), (6, 5, 16),
                       (6, 5, 8), (6, 5, 64), (65536, 65536, 32)):
        g = geom(rotate=1, L_high=lh, L_low=ll, q_heads=hq)
        assert sk._lib.semkv_cache_sizes(ctypes.byref(g), out) == sk.SEMKV_OK


def test_cache_sizes():
    s = sk.semkv_cache_sizes(geom())
    planes = 32 * 8 * 2
    assert s == [planes * 16384 * 43, planes * 16384 * 38, planes * 16384 * 4, planes * 16384 * 4,
                 16384 * 4, 16384 * 4, planes * 128 * 128 * 2, 128 * 4]


@pytest.mark.parametrize("bad,status", [
    (dict(head_dim=64), sk.SEMKV_EUNSUPPORTED),
    (dict(q_heads=30), sk.SEMKV_EINVAL),
    (dict(q_heads=8 * 16), sk.SEMKV_EUNSUPPORTED),
    (dict(L_low=2), sk.SEMKV_EINVAL),
    (dict(L_high=65537), sk.SEMKV_EINVAL),
    (dict(L_high=4, L_low=5), sk.SEMKV_EINVAL),
    (dict(cap_high=100), sk.SEMKV_EINVAL),
    (dict(block=0), sk.SEMKV_EINVAL),
    (dict(batch=0), sk.SEMKV_EINVAL),
    (dict(rotate=2), sk.SEMKV_EINVAL),
    (dict(rotate=1, q_heads=8 * 16), sk.SEMKV_EUNSUPPORTED),
])
def test_geometry_validation(bad, status):
    out = (ctypes.c_int64 * 8)()
    assert sk._lib.semkv_cache_sizes(ctypes.byref(geom(**bad)), out) == status


def test_workspace_query():
    g = geom()
    assert sk.semkv_workspace_bytes(g, 32, 32768) > 0
    # generation only: the block ranking's perm [batch][block] int32, then one
    # int32 per sequence for the ragged tail plan, each rounded to 256 bytes
    rnd = lambda x: (x + 255) // 256 * 256
    assert sk.semkv_workspace_bytes(g, 0, 0) == rnd(1 * 128 * 4) + rnd(1 * 4)
    assert sk._lib.semkv_workspace_bytes(ctypes.byref(g), 33, 10) < 0


def test_rank_argument_validation():
    f = sk._lib.semkv_rank_topr
    p = ctypes.c_void_p(0x1000)
    assert f(None, 1, 10, 10, 2, p, None, None) == sk.SEMKV_EINVAL          # null scores
    assert f(p, 1, 10, 10, 2, None, None, None) == sk.SEMKV_EINVAL          # null perm
    assert f(p, 1, 10, 10, 11, p, None, None) == sk.SEMKV_EINVAL            # k > n
    assert f(p, 1, 10, 9, 2, p, None, None) == sk.SEMKV_EINVAL              # ld < n
    assert f(p, 0, 10, 10, 2, p, None, None) == sk.SEMKV_EINVAL             # batch 0
    assert f(ctypes.c_void_p(0x1002), 1, 10, 10, 2, p, None, None) == sk.SEMKV_EINVAL  # misaligned


def fake_cache(**kw):
    g = geom(**kw)
    a = 0x100000
    return sk.semkv_cache(g=g, codes_high=a, codes_low=a, meta_high=a, meta_low=a, tok_high=a,
                          tok_low=a, tail_kv=a, tail_score=a, n_high=0, n_low=0, n_tail=0,
                          n_tokens=0)


def test_score_keynorm_validation_before_launch():
    f = sk._lib.semkv_score_keynorm
    p = ctypes.c_void_p(0x200000)
    st = (ctypes.c_int64 * 4)(32 * 8 * 1000 * 128, 8 * 1000 * 128, 1000 * 128, 128)
    bad = (ctypes.c_int64 * 4)(32 * 8 * 1000 * 128, 8 * 1000 * 128, 1000 * 128, 132)
    E = sk.SEMKV_EINVAL
    assert f(None, st, 1, 8, 1000, 28, 4, p, 1000, None) == E                 # null K
    assert f(ctypes.c_void_p(0x200008), st, 1, 8, 1000, 28, 4, p, 1000, None) == E   # K not 16-byte aligned
    assert f(p, bad, 1, 8, 1000, 28, 4, p, 1000, None) == E                  # stride not a multiple of 8
    assert f(p, None, 1, 8, 1000, 28, 4, p, 1000, None) == E                 # no strides
    assert f(p, st, 0, 8, 1000, 28, 4, p, 1000, None) == E                   # batch 0
    assert f(p, st, 65536, 8, 1000, 28, 4, p, 1000, None) == E               # batch too large
    assert f(p, st, 1, 0, 1000, 28, 4, p, 1000, None) == E                   # no heads
    assert f(p, st, 1, 8, 0, 28, 4, p, 1000, None) == E                      # n < 1
    assert f(p, st, 1, 8, 1000, -1, 4, p, 1000, None) == E                   # layer0 < 0
    assert f(p, st, 1, 8, 1000, 28, 0, p, 1000, None) == E                   # empty window
    assert f(p, st, 1, 8, 1000, 28, 4, None, 1000, None) == E                # null scores
    assert f(p, st, 1, 8, 1000, 28, 4, ctypes.c_void_p(0x200002), 1000, None) == E   # misaligned scores
    assert f(p, st, 1, 8, 1000, 28, 4, p, 999, None) == E                    # ld < n


def test_quantize_pack_validation_before_launch():
    f = sk._lib.semkv_quantize_pack
    c = fake_cache()
    p = ctypes.c_void_p(0x200000)
    st = (ctypes.c_int64 * 4)(32 * 8 * 32768 * 128, 8 * 32768 * 128, 32768 * 128, 128)
    # capacity: 16385 high rows do not fit
    assert f(ctypes.byref(c), p, p, st, 32768, p, 16385, None) == sk.SEMKV_ECAPACITY
    # k_high out of range, n < 1, null K, misaligned V, stride not a multiple of 8
    assert f(ctypes.byref(c), p, p, st, 32768, p, 32769, None) == sk.SEMKV_EINVAL
    assert f(ctypes.byref(c), p, p, st, 0, p, 0, None) == sk.SEMKV_EINVAL
    assert f(ctypes.byref(c), None, p, st, 100, p, 10, None) == sk.SEMKV_EINVAL
    assert f(ctypes.byref(c), p, ctypes.c_void_p(0x200008), st, 100, p, 10, None) == sk.SEMKV_EINVAL
    bad = (ctypes.c_int64 * 4)(*st)
    bad[3] = 100
    assert f(ctypes.byref(c), p, p, bad, 100, p, 10, None) == sk.SEMKV_EINVAL
    # a non-empty tail forbids prompt quantization; counters must be consistent
    c2 = fake_cache()
    c2.n_tail, c2.n_tokens = 3, 3
    assert f(ctypes.byref(c2), p, p, st, 100, p, 10, None) == sk.SEMKV_EINVAL
    c3 = fake_cache()
    c3.n_high = 5
    assert f(ctypes.byref(c3), p, p, st, 100, p, 10, None) == sk.SEMKV_EINVAL
    # misaligned pool pointer
    c4 = fake_cache()
    c4.codes_low = 0x100010
    assert f(ctypes.byref(c4), p, p, st, 100, p, 10, None) == sk.SEMKV_EINVAL


def test_decode_and_append_validation_before_launch():
    c = fake_cache()
    p = ctypes.c_void_p(0x200000)
    dec = sk._lib.semkv_decode_attn
    assert dec(ctypes.byref(c), p, 0, 1, 1.0, p, p, 1 << 30, None) == sk.SEMKV_EINVAL  # empty cache
    c.n_high, c.n_low, c.n_tokens = 100, 100, 200
    assert dec(ctypes.byref(c), p, 31, 2, 1.0, p, p, 1 << 30, None) == sk.SEMKV_EINVAL  # layers
    assert dec(ctypes.byref(c), p, 0, 1, 1.0, p, p, 16, None) == sk.SEMKV_EWORKSPACE
    assert dec(ctypes.byref(c), p, 0, 1, 1.0, p, None, 1 << 30, None) == sk.SEMKV_EWORKSPACE
    app = sk._lib.semkv_append_block
    st = (ctypes.c_int64 * 4)(0, 0, 0, 128)
    assert app(ctypes.byref(c), p, p, st, p, 1, 0.25, 0, p, 0, None) == sk.SEMKV_EWORKSPACE
    assert app(ctypes.byref(c), p, p, st, p, 1, 1.5, 0, p, 1 << 20, None) == sk.SEMKV_EINVAL
    full = fake_cache(cap_high=16, cap_low=16)
    # 128 new tokens complete a block needing 32 high rows: no room
    assert app(ctypes.byref(full), p, p, st, p, 128, 0.25, 0, p, 1 << 20, None) == sk.SEMKV_ECAPACITY


def test_status_strings():
    for s in range(-5, 1):
        assert sk.semkv_status_str(s)


def test_binding_rejects_layouts_the_kernels_cannot_read():
    """The binding checks shapes, dtypes and density before any call: the
    kernels read dense arrays (CPU tensors suffice, nothing is launched)."""
    import types
    import torch
    cache = types.SimpleNamespace(geom=types.SimpleNamespace(batch=2, q_heads=8))
    out = torch.zeros((2, 2, 8, 128), dtype=torch.float32)
    with pytest.raises(ValueError):
        sk.semkv_decode_merge(cache, out[:, 1:2])                        # strided view over batch
    with pytest.raises(ValueError):
        sk.semkv_decode_partials(cache, torch.zeros((2, 1, 8, 128), dtype=torch.float32))  # not fp16
    with pytest.raises(ValueError):
        sk.semkv_decode_attn(cache, torch.zeros((2, 1, 4, 128), dtype=torch.float16), out[:, :1])
    s = torch.zeros((2, 100), dtype=torch.float32)
    with pytest.raises(ValueError):
        sk.semkv_rank_topr(s[:, ::2], 10, torch.zeros((2, 50), dtype=torch.int32))
    with pytest.raises(ValueError):
        sk.semkv_rank_topr(s, 10, torch.zeros((2, 99), dtype=torch.int32))
    with pytest.raises(ValueError):
        sk.semkv_rank_topr(s, 10, torch.zeros((2, 100), dtype=torch.int64))


def test_binding_rejects_bad_quantize_and_append_inputs():
    """quantize_pack and append_block check dtype, geometry coverage and the
    perm / score layout before any call (CPU tensors: nothing is launched),
    and refuse host tensors even when their layout is right."""
    import types
    import torch
    geom = types.SimpleNamespace(batch=2, layers=3, kv_heads=2, q_heads=8)
    cache = types.SimpleNamespace(geom=geom, workspace=torch.zeros(256, dtype=torch.uint8))
    n = 40
    K = torch.zeros((2, 3, 2, n, 128), dtype=torch.float16)
    perm = torch.zeros((2, n), dtype=torch.int32)
    bad_inputs = [
        (K.float(), K.float(), perm),                                    # fp32 rows
        (K[:, :2], K[:, :2], perm),                                      # fewer layers than the cache
        (torch.zeros((2, 3, 4, n, 128), dtype=torch.float16),) * 2 + (perm,),   # more heads
        (K, K[..., :64], perm),                                          # V shape differs
        (K, K, perm.long()),                                             # int64 perm
        (K, K, perm[:, :n - 1]),                                         # perm too short
        (K, K, torch.zeros((2, 2 * n), dtype=torch.int32)[:, ::2]),      # strided perm
        (K, K, perm),                                                    # host tensors
    ]
    for k_, v_, p_ in bad_inputs:
        with pytest.raises(ValueError):
            sk.semkv_quantize_pack(cache, k_, v_, p_, 10)
    Kn = torch.zeros((2, 3, 2, 1, 128), dtype=torch.float16)
    s = torch.zeros((2, 1), dtype=torch.float32)
    bad_app = [
        (Kn, Kn, s.double()),                                            # fp64 scores
        (Kn, Kn, torch.zeros((2, 2), dtype=torch.float32)),              # wrong t_new
        (Kn, Kn, torch.zeros((1, 1), dtype=torch.float32)),              # wrong batch
        (Kn.float(), Kn.float(), s),                                     # fp32 rows
        (Kn[:, :1], Kn[:, :1], s),                                       # too few layers
        (Kn, Kn, s),                                                     # host tensors
    ]
    for k_, v_, s_ in bad_app:
        with pytest.raises(ValueError):
            sk.semkv_append_block(cache, k_, v_, s_, 0.25)


def test_ragged_validation_before_launch():
    """Ragged calls check their arguments on the host and launch nothing on
    a bad one (the pointers below are never dereferenced)."""
    c = fake_cache()
    p = ctypes.c_void_p(0x200000)
    seq = ctypes.c_void_p(0x300000)
    st = (ctypes.c_int64 * 4)(32 * 8 * 32768 * 128, 8 * 32768 * 128, 32768 * 128, 128)
    E = sk.SEMKV_EINVAL
    q = sk._lib.semkv_ragged_quantize_pack
    assert q(ctypes.byref(c), None, p, p, st, 100, p, 0.5, p, None) == E        # null seq
    assert q(ctypes.byref(c), ctypes.c_void_p(0x300004), p, p, st, 100, p, 0.5, p, None) == E
    assert q(ctypes.byref(c), seq, p, p, st, 0, p, 0.5, p, None) == E          # n_max < 1
    assert q(ctypes.byref(c), seq, p, p, st, 100, p, 1.5, p, None) == E        # r
    assert q(ctypes.byref(c), seq, p, p, st, 100, None, 0.5, p, None) == E     # null n_seq
    busy = fake_cache()
    busy.n_high, busy.n_tokens = 5, 5                                          # host counters in use
    assert q(ctypes.byref(busy), seq, p, p, st, 100, p, 0.5, p, None) == E
    a = sk._lib.semkv_ragged_append
    assert a(ctypes.byref(c), seq, p, p, st, p, p, None, 0.5, p, 16, None) == sk.SEMKV_EWORKSPACE
    assert a(ctypes.byref(c), seq, None, p, st, p, p, None, 0.5, p, 1 << 20, None) == E   # active, no K
    assert a(ctypes.byref(c), seq, p, p, st, p, ctypes.c_void_p(0x200002), None, 0.5, p, 1 << 20,
             None) == E                                                        # misaligned active
    d = sk._lib.semkv_ragged_decode_attn
    assert d(ctypes.byref(c), seq, p, 0, 1, 1.0, c.g.cap_high + 16, 0, p, p, 1 << 30, None) == E
    assert d(ctypes.byref(c), seq, p, 0, 1, 1.0, -1, 0, p, p, 1 << 30, None) == E
    assert d(ctypes.byref(c), seq, p, 0, 1, 1.0, 100, 100, p, p, 16, None) == sk.SEMKV_EWORKSPACE
    r = sk._lib.semkv_ragged_rank_topr
    assert r(p, 2, 100, 99, p, 0.5, p, None, None) == E                        # ld < n_max
    assert r(p, 2, 100, 100, None, 0.5, p, None, None) == E                    # null n_seq
    assert sk._lib.semkv_seq_reset(None, 2, None) == E
    assert sk._lib.semkv_seq_reset(seq, 0, None) == E


def test_score_hidden_delta_validation_before_launch():
    f = sk._lib.semkv_score_hidden_delta
    p = ctypes.c_void_p(0x200000)
    st = (ctypes.c_int64 * 3)(5 * 1000 * 4096, 1000 * 4096, 4096)
    E = sk.SEMKV_EINVAL
    assert f(None, st, 1, 5, 1000, 4096, p, 1000, None) == E               # null h
    assert f(ctypes.c_void_p(0x200008), st, 1, 5, 1000, 4096, p, 1000, None) == E   # misaligned h
    assert f(p, st, 1, 1, 1000, 4096, p, 1000, None) == E                  # one state: no update
    assert f(p, st, 1, 10, 1000, 4096, p, 1000, None) == E                 # more than 8 layers
    assert f(p, st, 1, 5, 1000, 4100, p, 1000, None) == E                  # d not a multiple of 8
    assert f(p, st, 1, 5, 1000, 4096, p, 999, None) == E                   # ld < n
    assert f(p, st, 0, 5, 1000, 4096, p, 1000, None) == E                  # batch
    bad = (ctypes.c_int64 * 3)(*st)
    bad[2] = 100
    assert f(p, bad, 1, 5, 1000, 4096, p, 1000, None) == E                 # stride not a multiple of 8
