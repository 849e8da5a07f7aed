"""Thin Python binding of libsemkv.so (include/semkv.h).

Argument marshalling only: every function forwards device pointers of torch
tensors and the current (or given) HIP stream to the C entry point of the
same name and raises SemKVError on a non-zero status.  No arithmetic of the
method happens here; there is no CPU fallback -- importing this module fails
if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsemkv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python -m kv_cache_mixed_top_amd.build` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

c_i32, c_i64, c_p, c_f32, c_f64 = (ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p,
                                   ctypes.c_float, ctypes.c_double)

SEMKV_OK, SEMKV_EINVAL, SEMKV_EUNSUPPORTED, SEMKV_ECAPACITY, SEMKV_EWORKSPACE, SEMKV_EHIP = \
    0, -1, -2, -3, -4, -5


class semkv_geom(ctypes.Structure):
    _fields_ = [("batch", c_i32), ("layers", c_i32), ("kv_heads", c_i32), ("q_heads", c_i32),
                ("head_dim", c_i32), ("L_high", c_i32), ("L_low", c_i32), ("block", c_i32),
                ("cap_high", c_i64), ("cap_low", c_i64), ("rotate", c_i32)]


class semkv_cache(ctypes.Structure):
    _fields_ = [("g", semkv_geom),
                ("codes_high", c_p), ("codes_low", c_p), ("meta_high", c_p), ("meta_low", c_p),
                ("tok_high", c_p), ("tok_low", c_p), ("tail_kv", c_p), ("tail_score", c_p),
                ("n_high", c_i64), ("n_low", c_i64), ("n_tail", c_i64), ("n_tokens", c_i64)]


_SIGS = {
    "semkv_row_bytes": (c_i64, [c_i32]),
    "semkv_topr_count": (c_i64, [c_i64, c_f64]),
    "semkv_cache_sizes": (c_i32, [ctypes.POINTER(semkv_geom), ctypes.POINTER(c_i64)]),
    "semkv_workspace_bytes": (c_i64, [ctypes.POINTER(semkv_geom), c_i32, c_i64]),
    "semkv_score_keynorm": (c_i32, [c_p, ctypes.POINTER(c_i64), c_i32, c_i32, c_i64, c_i32, c_i32,
                                    c_p, c_i64, c_p]),
    "semkv_score_hidden_delta": (c_i32, [c_p, ctypes.POINTER(c_i64), c_i32, c_i32, c_i64, c_i32,
                                         c_p, c_i64, c_p]),
    "semkv_rank_topr": (c_i32, [c_p, c_i32, c_i64, c_i64, c_i64, c_p, c_p, c_p]),
    "semkv_quantize_pack": (c_i32, [ctypes.POINTER(semkv_cache), c_p, c_p,
                                    ctypes.POINTER(c_i64), c_i64, c_p, c_i64, c_p]),
    "semkv_append_block": (c_i32, [ctypes.POINTER(semkv_cache), c_p, c_p, ctypes.POINTER(c_i64),
                                   c_p, c_i32, c_f64, c_i32, c_p, c_i64, c_p]),
    "semkv_decode_attn": (c_i32, [ctypes.POINTER(semkv_cache), c_p, c_i32, c_i32, c_f32, c_p,
                                  c_p, c_i64, c_p]),
    "semkv_decode_partials": (c_i32, [ctypes.POINTER(semkv_cache), c_p, c_i32, c_i32, c_f32,
                                      c_p, c_i64, c_p]),
    "semkv_decode_merge": (c_i32, [ctypes.POINTER(semkv_cache), c_i32, c_p, c_p, c_i64, c_p]),
    "semkv_decode_attn_noalloc": (c_i32, [ctypes.POINTER(semkv_cache), c_p, c_i32, c_i32, c_f32,
                                          c_p, c_p]),
    "semkv_decode_noalloc_scratch_bytes": (c_i64, []),
    "semkv_dequantize_rows": (c_i32, [ctypes.POINTER(semkv_cache), c_i32, c_i32, c_i64, c_i64,
                                      c_p, c_p]),
    "semkv_seq_reset": (c_i32, [c_p, c_i32, c_p]),
    "semkv_ragged_rank_topr": (c_i32, [c_p, c_i32, c_i64, c_i64, c_p, c_f64, c_p, c_p, c_p]),
    "semkv_ragged_quantize_pack": (c_i32, [ctypes.POINTER(semkv_cache), c_p, c_p, c_p,
                                           ctypes.POINTER(c_i64), c_i64, c_p, c_f64, c_p, c_p]),
    "semkv_ragged_append": (c_i32, [ctypes.POINTER(semkv_cache), c_p, c_p, c_p,
                                    ctypes.POINTER(c_i64), c_p, c_p, c_p, c_f64, c_p, c_i64, c_p]),
    "semkv_ragged_decode_attn": (c_i32, [ctypes.POINTER(semkv_cache), c_p, c_p, c_i32, c_i32, c_f32,
                                         c_i64, c_i64, c_p, c_p, c_i64, c_p]),
    "semkv_sync_check": (c_i32, [c_p]),
    "semkv_status_str": (ctypes.c_char_p, [c_i32]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


class SemKVError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {_lib.semkv_status_str(status).decode()} ({status})")


def _check(fn, status):
    if status != SEMKV_OK:
        raise SemKVError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _strides(t):
    """Element strides (batch, layer, head, token) of a [B][layers][kv][n][128] view."""
    if t.dim() != 5 or t.shape[-1] != 128 or t.stride(-1) != 1:
        raise ValueError("K/V must be [batch][layers][kv_heads][tokens][128] with unit-stride d")
    return (c_i64 * 4)(*[t.stride(i) for i in range(4)])


def _nbytes(t):
    return t.numel() * t.element_size()


def _on_device(*ts):
    """The C entry points take device pointers: host tensors are refused here,
    after the layout checks (which need no device)."""
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors passed to the library must live on the GPU")


def _kv_rows(cache, K, V, what):
    """K and V: fp16 [batch][layers][kv_heads][tokens][128] views with unit-
    stride d that share shape and strides, covering the cache's geometry."""
    g = cache.geom
    for t in (K, V):
        if t.dtype != torch.float16:
            raise ValueError(f"{what} must be fp16")
        if t.dim() != 5 or tuple(t.shape[:3]) != (g.batch, g.layers, g.kv_heads):
            raise ValueError(f"{what} must be [{g.batch}][{g.layers}][{g.kv_heads}][tokens][128]")
    if V.shape != K.shape or tuple(V.stride()) != tuple(K.stride()):
        raise ValueError(f"{what}: K and V must share shape and strides")
    return _strides(K)


# ------------------------------------------------------------------ host-only

def semkv_row_bytes(L: int) -> int:
    return _lib.semkv_row_bytes(L)


def semkv_topr_count(n: int, r: float) -> int:
    return _lib.semkv_topr_count(n, r)


def semkv_cache_sizes(geom: semkv_geom):
    out = (c_i64 * 8)()
    _check("semkv_cache_sizes", _lib.semkv_cache_sizes(ctypes.byref(geom), out))
    return list(out)


def semkv_workspace_bytes(geom: semkv_geom, nlayers: int, max_tokens: int) -> int:
    v = _lib.semkv_workspace_bytes(ctypes.byref(geom), nlayers, max_tokens)
    if v < 0:
        raise SemKVError("semkv_workspace_bytes", SEMKV_EINVAL)
    return v


# ------------------------------------------------------------------ device calls

def semkv_score_keynorm(K, scores, layer0, nlayers, stream=None):
    """K fp16 [B][layers][kv][n][128] (any strides with d contiguous); scores fp32 [B][ld] out."""
    if layer0 < 0 or nlayers < 1 or layer0 + nlayers > K.shape[1]:
        raise ValueError("layer window outside K")
    if K.dtype != torch.float16:
        raise ValueError("K must be fp16")
    if (scores.dtype != torch.float32 or scores.dim() != 2 or scores.shape[0] != K.shape[0]
            or scores.shape[1] < K.shape[3] or scores.stride(1) != 1):
        raise ValueError("scores must be fp32 [B][>= n] with unit stride")
    strides = _strides(K)
    _on_device(K, scores)
    _check("semkv_score_keynorm",
           _lib.semkv_score_keynorm(_ptr(K), strides, K.shape[0], K.shape[2], K.shape[3],
                                    layer0, nlayers, _ptr(scores), scores.stride(0),
                                    _stream(stream)))


def semkv_score_hidden_delta(H, scores, stream=None):
    """H fp16 [B][states][n][d] (d contiguous, other strides multiples of 8);
    scores fp32 [B][>= n] out: sum over consecutive states of ||h_j - h_{j-1}||."""
    if H.dtype != torch.float16 or H.dim() != 4 or H.stride(3) != 1:
        raise ValueError("H must be fp16 [B][states][n][d] with d contiguous")
    B, S1, n, d = H.shape
    if (scores.dtype != torch.float32 or scores.dim() != 2 or scores.shape[0] != B
            or scores.shape[1] < n or scores.stride(1) != 1):
        raise ValueError("scores must be fp32 [B][>= n] with unit stride")
    strides = (c_i64 * 3)(H.stride(0), H.stride(1), H.stride(2))
    _on_device(H, scores)
    _check("semkv_score_hidden_delta",
           _lib.semkv_score_hidden_delta(_ptr(H), strides, B, S1, n, d, _ptr(scores), scores.stride(0),
                                         _stream(stream)))


def semkv_rank_topr(scores, k, perm, mask=None, n=None, stream=None):
    """scores fp32 [B][ld]; perm int32 [B][n] out; mask uint32-as-int32 [B][ceil(n/32)] out."""
    batch = scores.shape[0]
    n = scores.shape[1] if n is None else n
    if scores.dtype != torch.float32 or scores.dim() != 2 or scores.stride(1) != 1 or n > scores.shape[1]:
        raise ValueError("scores must be fp32 [B][>= n] with unit stride")
    if (perm.dtype != torch.int32 or tuple(perm.shape) != (batch, n) or not perm.is_contiguous()):
        raise ValueError("perm must be a contiguous int32 [B][n] tensor")
    if mask is not None and (mask.dtype != torch.int32 or tuple(mask.shape) != (batch, (n + 31) // 32)
                             or not mask.is_contiguous()):
        raise ValueError("mask must be a contiguous int32 [B][ceil(n/32)] tensor")
    _on_device(scores, perm, mask)
    _check("semkv_rank_topr", _lib.semkv_rank_topr(_ptr(scores), batch, n, scores.stride(0), k,
                                                   _ptr(perm), _ptr(mask), _stream(stream)))


def semkv_quantize_pack(cache: "SemKVCache", K, V, perm, k_high, stream=None):
    """K, V fp16 [batch][layers][kv][n][128] (d contiguous); perm int32 [batch][n]."""
    strides = _kv_rows(cache, K, V, "K/V")
    n = K.shape[3]
    if (perm.dtype != torch.int32 or tuple(perm.shape) != (cache.geom.batch, n)
            or not perm.is_contiguous()):
        raise ValueError("perm must be a contiguous int32 [batch][n] tensor")
    _on_device(K, V, perm)
    _check("semkv_quantize_pack",
           _lib.semkv_quantize_pack(ctypes.byref(cache.c), _ptr(K), _ptr(V), strides, n,
                                    _ptr(perm), k_high, _stream(stream)))


def semkv_append_block(cache: "SemKVCache", K_new, V_new, score_new, r, flush=False,
                       workspace=None, stream=None):
    """K_new/V_new fp16 [B][layers][kv][t_new][128] (or None with flush); score_new [B][t_new]."""
    ws = cache.workspace if workspace is None else workspace
    if K_new is None:
        _on_device(ws)
        _check("semkv_append_block",
               _lib.semkv_append_block(ctypes.byref(cache.c), None, None, None, None, 0, r,
                                       int(bool(flush)), _ptr(ws), _nbytes(ws), _stream(stream)))
        return
    strides = _kv_rows(cache, K_new, V_new, "K_new/V_new")
    t_new = K_new.shape[3]
    if (score_new.dtype != torch.float32 or tuple(score_new.shape) != (cache.geom.batch, t_new)
            or not score_new.is_contiguous()):
        raise ValueError("score_new must be a contiguous fp32 [batch][t_new] tensor")
    _on_device(K_new, V_new, score_new, ws)
    _check("semkv_append_block",
           _lib.semkv_append_block(ctypes.byref(cache.c), _ptr(K_new), _ptr(V_new),
                                   strides, _ptr(score_new), t_new, r, int(bool(flush)),
                                   _ptr(ws), _nbytes(ws), _stream(stream)))


def _dense(t, name, dtype, cache):
    """The kernels read q and write out as dense [B][nl][Hq][128] arrays."""
    g = cache.geom
    if (t.dtype != dtype or t.dim() != 4 or t.shape[0] != g.batch or t.shape[2] != g.q_heads
            or t.shape[3] != 128 or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} [batch][nl][q_heads][128] tensor")
    _on_device(t)


def semkv_decode_attn(cache: "SemKVCache", q, out, layer0=0, sm_scale=1.0, workspace=None,
                      stream=None):
    """q fp16 [B][nl][Hq][128]; out fp32 [B][nl][Hq][128]."""
    _dense(q, "q", torch.float16, cache)
    _dense(out, "out", torch.float32, cache)
    if out.shape[1] != q.shape[1]:
        raise ValueError("q and out must cover the same layers")
    ws = cache.workspace if workspace is None else workspace
    _on_device(ws)
    _check("semkv_decode_attn",
           _lib.semkv_decode_attn(ctypes.byref(cache.c), _ptr(q), layer0, q.shape[1], sm_scale,
                                  _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream)))


def semkv_decode_attn_noalloc(cache: "SemKVCache", q, out, layer0=0, sm_scale=1.0, stream=None):
    """semkv_decode_attn with the partials in the library's static device
    scratch (no workspace argument, nothing allocated)."""
    _dense(q, "q", torch.float16, cache)
    _dense(out, "out", torch.float32, cache)
    if out.shape[1] != q.shape[1]:
        raise ValueError("q and out must cover the same layers")
    _check("semkv_decode_attn_noalloc",
           _lib.semkv_decode_attn_noalloc(ctypes.byref(cache.c), _ptr(q), layer0, q.shape[1],
                                          sm_scale, _ptr(out), _stream(stream)))


def semkv_decode_noalloc_scratch_bytes() -> int:
    return _lib.semkv_decode_noalloc_scratch_bytes()


def semkv_decode_partials(cache: "SemKVCache", q, layer0=0, sm_scale=1.0, workspace=None,
                          stream=None):
    _dense(q, "q", torch.float16, cache)
    ws = cache.workspace if workspace is None else workspace
    _on_device(ws)
    _check("semkv_decode_partials",
           _lib.semkv_decode_partials(ctypes.byref(cache.c), _ptr(q), layer0, q.shape[1],
                                      sm_scale, _ptr(ws), _nbytes(ws), _stream(stream)))


def semkv_decode_merge(cache: "SemKVCache", out, workspace=None, stream=None):
    _dense(out, "out", torch.float32, cache)
    ws = cache.workspace if workspace is None else workspace
    _on_device(ws)
    _check("semkv_decode_merge",
           _lib.semkv_decode_merge(ctypes.byref(cache.c), out.shape[1], _ptr(out), _ptr(ws),
                                   _nbytes(ws), _stream(stream)))


def semkv_dequantize_rows(cache: "SemKVCache", high: bool, layer, row0, nrows, out,
                          stream=None):
    """out fp32 [batch][kv_heads][2][nrows][128]: rows row0 .. row0+nrows-1 of one
    layer of the high (or low) pool, reconstructed."""
    g = cache.geom
    if (out.dtype != torch.float32 or tuple(out.shape) != (g.batch, g.kv_heads, 2, nrows, 128)
            or not out.is_contiguous()):
        raise ValueError("out must be a contiguous fp32 [batch][kv_heads][2][nrows][128] tensor")
    _on_device(out)
    _check("semkv_dequantize_rows",
           _lib.semkv_dequantize_rows(ctypes.byref(cache.c), 0 if high else 1, layer, row0, nrows,
                                      _ptr(out), _stream(stream)))


# ------------------------------------------------------------------ ragged batches

SEQ_WORDS = 8          # int64 counters per sequence: n_high, n_low, n_tail, n_tokens, status
SEQ_HIGH, SEQ_LOW, SEQ_TAIL, SEQ_TOKENS, SEQ_STATUS = range(5)


def _seq(cache, seq):
    if (seq.dtype != torch.int64 or tuple(seq.shape) != (cache.geom.batch, SEQ_WORDS)
            or not seq.is_contiguous()):
        raise ValueError(f"seq must be a contiguous int64 [batch][{SEQ_WORDS}] tensor")
    _on_device(seq)


def _per_seq_i32(cache, t, name):
    if t is None:
        return
    if t.dtype != torch.int32 or tuple(t.shape) != (cache.geom.batch,) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 [batch] tensor")
    _on_device(t)


def semkv_seq_reset(seq, stream=None):
    if seq.dtype != torch.int64 or seq.dim() != 2 or seq.shape[1] != SEQ_WORDS or not seq.is_contiguous():
        raise ValueError(f"seq must be a contiguous int64 [batch][{SEQ_WORDS}] tensor")
    _on_device(seq)
    _check("semkv_seq_reset", _lib.semkv_seq_reset(_ptr(seq), seq.shape[0], _stream(stream)))


def semkv_ragged_rank_topr(scores, n_seq, r, perm, mask=None, stream=None):
    """scores fp32 [B][>= n_max]; n_seq int32 [B]; perm int32 [B][n_max] out."""
    batch, n_max = perm.shape
    if scores.dtype != torch.float32 or scores.dim() != 2 or scores.stride(1) != 1 or scores.shape[1] < n_max:
        raise ValueError("scores must be fp32 [B][>= n_max] with unit stride")
    if perm.dtype != torch.int32 or not perm.is_contiguous() or scores.shape[0] != batch:
        raise ValueError("perm must be a contiguous int32 [B][n_max] tensor")
    if n_seq.dtype != torch.int32 or tuple(n_seq.shape) != (batch,) or not n_seq.is_contiguous():
        raise ValueError("n_seq must be a contiguous int32 [B] tensor")
    if mask is not None and (mask.dtype != torch.int32 or tuple(mask.shape) != (batch, (n_max + 31) // 32)
                             or not mask.is_contiguous()):
        raise ValueError("mask must be a contiguous int32 [B][ceil(n_max/32)] tensor")
    _on_device(scores, n_seq, perm, mask)
    _check("semkv_ragged_rank_topr",
           _lib.semkv_ragged_rank_topr(_ptr(scores), batch, n_max, scores.stride(0), _ptr(n_seq), r,
                                       _ptr(perm), _ptr(mask), _stream(stream)))


def semkv_ragged_quantize_pack(cache: "SemKVCache", seq, K, V, n_seq, r, perm, stream=None):
    """K, V fp16 [batch][layers][kv][n_max][128]; n_seq int32 [batch]; perm int32 [batch][n_max]."""
    strides = _kv_rows(cache, K, V, "K/V")
    n_max = K.shape[3]
    _seq(cache, seq)
    _per_seq_i32(cache, n_seq, "n_seq")
    if perm.dtype != torch.int32 or tuple(perm.shape) != (cache.geom.batch, n_max) or not perm.is_contiguous():
        raise ValueError("perm must be a contiguous int32 [batch][n_max] tensor")
    _on_device(K, V, perm)
    _check("semkv_ragged_quantize_pack",
           _lib.semkv_ragged_quantize_pack(ctypes.byref(cache.c), _ptr(seq), _ptr(K), _ptr(V), strides,
                                           n_max, _ptr(n_seq), r, _ptr(perm), _stream(stream)))


def semkv_ragged_append(cache: "SemKVCache", seq, K_new, V_new, score_new, active, r, flush=None,
                        workspace=None, stream=None):
    """One token per active sequence: K_new/V_new fp16 [batch][layers][kv][1][128], score_new fp32
    [batch], active / flush int32 [batch] (either may be None)."""
    _seq(cache, seq)
    _per_seq_i32(cache, active, "active")
    _per_seq_i32(cache, flush, "flush")
    ws = cache.workspace if workspace is None else workspace
    _on_device(ws)
    if active is None:
        _check("semkv_ragged_append",
               _lib.semkv_ragged_append(ctypes.byref(cache.c), _ptr(seq), None, None, None, None, None,
                                        _ptr(flush), r, _ptr(ws), _nbytes(ws), _stream(stream)))
        return
    strides = _kv_rows(cache, K_new, V_new, "K_new/V_new")
    if K_new.shape[3] != 1:
        raise ValueError("K_new/V_new hold one token per sequence")
    if (score_new.dtype != torch.float32 or tuple(score_new.shape) != (cache.geom.batch,)
            or not score_new.is_contiguous()):
        raise ValueError("score_new must be a contiguous fp32 [batch] tensor")
    _on_device(K_new, V_new, score_new)
    _check("semkv_ragged_append",
           _lib.semkv_ragged_append(ctypes.byref(cache.c), _ptr(seq), _ptr(K_new), _ptr(V_new), strides,
                                    _ptr(score_new), _ptr(active), _ptr(flush), r, _ptr(ws), _nbytes(ws),
                                    _stream(stream)))


def semkv_ragged_decode_attn(cache: "SemKVCache", seq, q, out, max_high, max_low, layer0=0, sm_scale=1.0,
                             workspace=None, stream=None):
    """q fp16 [B][nl][Hq][128]; out fp32 [B][nl][Hq][128]; max_high / max_low bound the
    sequences' pool rows."""
    _seq(cache, seq)
    _dense(q, "q", torch.float16, cache)
    _dense(out, "out", torch.float32, cache)
    if out.shape[1] != q.shape[1]:
        raise ValueError("q and out must cover the same layers")
    ws = cache.workspace if workspace is None else workspace
    _on_device(ws)
    _check("semkv_ragged_decode_attn",
           _lib.semkv_ragged_decode_attn(ctypes.byref(cache.c), _ptr(seq), _ptr(q), layer0, q.shape[1],
                                         sm_scale, max_high, max_low, _ptr(out), _ptr(ws), _nbytes(ws),
                                         _stream(stream)))


def semkv_sync_check(stream=None):
    _check("semkv_sync_check", _lib.semkv_sync_check(_stream(stream)))


def semkv_status_str(status: int) -> str:
    return _lib.semkv_status_str(status).decode()


# ------------------------------------------------------------------ cache holder

class SemKVCache:
    """Device buffers of one cache, allocated with torch, and its C struct.

    The buffers are plain tensors (views of the C layout in include/semkv.h);
    the host counters live in the struct and are advanced by the C calls.
    """

    def __init__(self, batch, layers, kv_heads, q_heads, L_high, L_low, cap_high, cap_low,
                 block=128, device="cuda", max_decode_layers=None, max_tokens=None,
                 rotate=False):
        g = semkv_geom(batch=batch, layers=layers, kv_heads=kv_heads, q_heads=q_heads,
                       head_dim=128, L_high=L_high, L_low=L_low, block=block,
                       cap_high=cap_high, cap_low=cap_low, rotate=int(bool(rotate)))
        sizes = semkv_cache_sizes(g)
        self.geom = g
        dev = torch.device(device)
        self.codes_high = torch.zeros(sizes[0], dtype=torch.uint8, device=dev)
        self.codes_low = torch.zeros(sizes[1], dtype=torch.uint8, device=dev)
        self.meta_high = torch.zeros(sizes[2] // 2, dtype=torch.int16, device=dev)
        self.meta_low = torch.zeros(sizes[3] // 2, dtype=torch.int16, device=dev)
        self.tok_high = torch.full((sizes[4] // 4,), -1, dtype=torch.int32, device=dev)
        self.tok_low = torch.full((sizes[5] // 4,), -1, dtype=torch.int32, device=dev)
        self.tail_kv = torch.zeros(sizes[6] // 2, dtype=torch.float16, device=dev)
        self.tail_score = torch.zeros(sizes[7] // 4, dtype=torch.float32, device=dev)
        nl = layers if max_decode_layers is None else max_decode_layers
        mt = cap_high + cap_low + block if max_tokens is None else max_tokens
        self.workspace = torch.empty(semkv_workspace_bytes(g, nl, mt), dtype=torch.uint8,
                                     device=dev)
        self.c = semkv_cache(g=g,
                             codes_high=self.codes_high.data_ptr() or None,
                             codes_low=self.codes_low.data_ptr() or None,
                             meta_high=self.meta_high.data_ptr() or None,
                             meta_low=self.meta_low.data_ptr() or None,
                             tok_high=self.tok_high.data_ptr() or None,
                             tok_low=self.tok_low.data_ptr() or None,
                             tail_kv=self.tail_kv.data_ptr(),
                             tail_score=self.tail_score.data_ptr(),
                             n_high=0, n_low=0, n_tail=0, n_tokens=0)

    # counters
    @property
    def n_high(self):
        return self.c.n_high

    @property
    def n_low(self):
        return self.c.n_low

    @property
    def n_tail(self):
        return self.c.n_tail

    @property
    def n_tokens(self):
        return self.c.n_tokens

    def reset(self):
        self.c.n_high = self.c.n_low = self.c.n_tail = self.c.n_tokens = 0

    # shaped views of the C layout (for tests and checkpointing)
    def codes_view(self, high: bool):
        g = self.geom
        L = g.L_high if high else g.L_low
        cap = g.cap_high if high else g.cap_low
        t = self.codes_high if high else self.codes_low
        return t.view(g.batch, g.layers, g.kv_heads, 2, cap, semkv_row_bytes(L))

    def meta_view(self, high: bool):
        g = self.geom
        cap = g.cap_high if high else g.cap_low
        t = self.meta_high if high else self.meta_low
        return t.view(g.batch, g.layers, g.kv_heads, 2, cap, 2)

    def tok_view(self, high: bool):
        g = self.geom
        cap = g.cap_high if high else g.cap_low
        return (self.tok_high if high else self.tok_low).view(g.batch, cap)

    def tail_view(self):
        g = self.geom
        return self.tail_kv.view(g.batch, g.layers, g.kv_heads, 2, g.block, 128)

    def state_dict(self):
        """Buffers and counters; load_state_dict restores an identical cache."""
        d = {k: getattr(self, k).clone() for k in ("codes_high", "codes_low", "meta_high",
                                                   "meta_low", "tok_high", "tok_low",
                                                   "tail_kv", "tail_score")}
        d["counters"] = (self.c.n_high, self.c.n_low, self.c.n_tail, self.c.n_tokens)
        return d

    def load_state_dict(self, d):
        for k in ("codes_high", "codes_low", "meta_high", "meta_low", "tok_high", "tok_low",
                  "tail_kv", "tail_score"):
            getattr(self, k).copy_(d[k])
        self.c.n_high, self.c.n_low, self.c.n_tail, self.c.n_tokens = d["counters"]
