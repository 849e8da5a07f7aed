"""CPU oracle for the SemKV mixed-precision KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, obviously-correct
statement of what the hot path computes.  It is imported only by the tests,
by ``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of
``bench.py``; the product path (the HIP library and its Python binding) never
imports, links or calls it, and it shares no code, table or helper with that
path.  Everything here is numpy in float64 (fp16 values are exact in float64).

Source pages (cited by title and figure/table; the text is not quoted):
  "SemKV: Semantic Mixed-Precision KV Cache Quantization Guided by the Quality
  Cliff for Long-Context LLM Inference" -- abbreviated *SemKV* below -- its
  figure/table captions (Figs. 1-6, Tables 2, 6, 7) and its abstract.

The pages give captions and an abstract only; where they leave a step open,
the reading used here is the plainest one that the rest supports, marked
"(open on the pages)" below.  In short:

  * k = floor(r*n + 1/2)                                 (open on the pages)
  * ties in score go to the lower token index; -0 == +0; NaN ranks below
    every number                                         (open on the pages)
  * one top-r set per sequence, shared by every layer, KV head, K and V
                                                         (SemKV Fig. 5)
  * a quantization row is the 128 values of one (token, layer, KV head,
    K-or-V); two fp16 scalars per row: scale then min   (SemKV Table 6)
  * scale = smallest fp16 >= (max-min)/(L-1); codes = round-half-even of
    (x-min)/scale, clamped to [0, L-1]                   (open on the pages)
  * packing: g codes of base L per b-bit field, first code in the least
    significant digit, fields LSB-first in a little-endian bit stream
    (our layout; the pages fix only the rates of SemKV Table 6)
  * optional Hadamard rotation of every row before quantization (SemKV
    Table 2 lists one in the default quantizer; which Hadamard matrix and in
    what precision is open on the pages): the normalized Sylvester H_128
    without sign changes, applied in float32 by seven butterfly stages in
    index-bit order, then one multiply by float32(1/sqrt(128)); the minimum
    of a rotated row is rounded down to fp16.  Decode rotates the query and
    rotates the output back (H is symmetric and orthogonal).

Parity pins for every function live in tests/test_oracle_pins.py,
tests/test_oracle_props.py and the other tests/test_oracle_*.py files.  One
reading is "parity unpinned" beyond a bound: the float32 butterfly order of
rotate_rows_f32 (and hence the exact bits of the rotated codes that
quantize_rows_rotated derives from it) is a convention of ours; the pages fix
no order or precision, so it is pinned only to within its rounding bound of
the exact float64 rotation, not bit for bit.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 128

# --------------------------------------------------------------------------
# Scoring by key norm (SemKV Fig. 2: one model-internal indicator gives a
# per-token score; SemKV Table 3 lists the key-norm indicator among the
# variants; its exact form and layer window are open on the pages).
# Reading: the score of token t is the sum, over the layers of a window and
# every KV head, of the Euclidean norm of t's key row.  Only the order of the
# scores matters to the ranking (SemKV Fig. 2), so no normalisation.
# --------------------------------------------------------------------------


def score_keynorm(K: np.ndarray, layer0: int, nlayers: int) -> np.ndarray:
    """K fp16 [B][layers][kv][n][128] -> float64 [B][n]:
    score[b, t] = sum over layers layer0 .. layer0+nlayers-1 and KV heads h
    of sqrt(sum_d K[b, layer, h, t, d]^2)."""
    K = np.asarray(K, dtype=np.float16).astype(np.float64)
    rows = K[:, layer0:layer0 + nlayers]                  # [B][nl][kv][n][128]
    norms = np.sqrt(np.sum(rows * rows, axis=-1))        # [B][nl][kv][n]
    return norms.sum(axis=(1, 2))


# --------------------------------------------------------------------------
# Scoring by hidden-state delta norm (SemKV Table 2: the default indicator is
# the hidden-state delta norm over the last 4 layers; Fig. 10: it costs O(1)
# per token, being read from the token's own hidden states).  Reading (the
# formula is open on the pages): with h_0 .. h_S the hidden states of token
# t entering and leaving the last S layers (S = 4), the score is the sum over
# those layers of the Euclidean norm of the layer's update, sum_{j=1..S}
# ||h_j[t] - h_{j-1}[t]||_2.  Only the order matters to the ranking.
# --------------------------------------------------------------------------


def score_hidden_delta(H: np.ndarray) -> np.ndarray:
    """H fp16 [B][S+1][n][d] (hidden states h_0 .. h_S per token) -> float64
    [B][n]: score[b, t] = sum_{j=1..S} sqrt(sum_k (H[b,j,t,k] - H[b,j-1,t,k])^2)."""
    H = np.asarray(H, dtype=np.float16).astype(np.float64)
    if H.ndim != 4 or H.shape[1] < 2:
        raise ValueError("need H [B][S+1][n][d] with S >= 1")
    D = H[:, 1:] - H[:, :-1]                               # [B][S][n][d], exact in float64
    return np.sqrt(np.sum(D * D, axis=-1)).sum(axis=1)


# --------------------------------------------------------------------------
# Rank (SemKV Fig. 2: ranking within each prompt, no score normalisation;
#       SemKV Fig. 4: the top-r tokens form the high-precision set H, no
#       threshold is estimated; SemKV Fig. 5: one assignment per token,
#       broadcast over layers and KV heads).
# --------------------------------------------------------------------------


def topr_count(n: int, r: float) -> int:
    """Number of high-precision tokens for a fraction r of n tokens.

    Open on the pages; our reading: round r*n to the nearest integer, halves
    up, in float64.
    """
    if n < 0 or not (0.0 <= r <= 1.0):
        raise ValueError("need n >= 0 and 0 <= r <= 1")
    return int(math.floor(float(r) * float(n) + 0.5))


def rank_order(scores: np.ndarray) -> np.ndarray:
    """Token indices ordered best-first: score descending, index ascending.

    Scores compare as IEEE numbers (so -0 equals +0); every NaN ranks below
    every number and NaNs tie among themselves (open on the pages).
    """
    s = np.asarray(scores, dtype=np.float64).ravel()
    n = s.shape[0]
    is_nan = np.isnan(s)
    neg = np.where(is_nan, 0.0, -s)          # ascending in -s == descending in s
    neg = neg + 0.0                          # -0 -> +0 (both compare equal anyway)
    idx = np.arange(n)
    # np.lexsort sorts by the LAST key first: NaN flag, then -score, then index.
    return np.lexsort((idx, neg, is_nan))


def rank_topr(scores: np.ndarray, k: int):
    """Top-k set of one sequence.

    Returns (perm, mask):
      perm  int32[n]  = H in ascending token order, then the rest ascending
      mask  uint32[ceil(n/32)], bit (t % 32) of word t // 32 set iff t in H
    """
    s = np.asarray(scores).ravel()
    n = s.shape[0]
    if not (0 <= k <= n):
        raise ValueError("need 0 <= k <= n")
    order = rank_order(s)
    in_h = np.zeros(n, dtype=bool)
    in_h[order[:k]] = True
    idx = np.arange(n)
    perm = np.concatenate([idx[in_h], idx[~in_h]]).astype(np.int32)
    nwords = (n + 31) // 32
    flags = np.zeros(nwords * 32, dtype=np.uint64)
    flags[:n] = in_h
    # word w = sum over i < 32 of flag[32 w + i] * 2^i
    mask = (flags.reshape(nwords, 32) << np.arange(32, dtype=np.uint64)).sum(axis=1)
    return perm, mask.astype(np.uint32)


def rank_topr_batch(scores: np.ndarray, k: int):
    """rank_topr for every row of a [B][n] score matrix."""
    s = np.asarray(scores)
    perms, masks = zip(*(rank_topr(s[b], k) for b in range(s.shape[0])))
    return np.stack(perms), np.stack(masks)


# --------------------------------------------------------------------------
# Quantize one row (SemKV Table 2: integer-level scalar quantizer; Table 6:
# affine base, two scalars per 128-value row, code bits log2-like per level
# count; Fig. 1: two precisions b_high / b_low on the level grid).
# --------------------------------------------------------------------------


def scale_fp16_ceil(lo: np.ndarray, hi: np.ndarray, L: int) -> np.ndarray:
    """Smallest fp16 value >= (hi - lo) / (L - 1), elementwise (open on the
    pages: a ceiling, so that no code is clipped).

    hi - lo is exact in float64 (fp16 operands); the correctly rounded float64
    quotient has the same fp16 ceiling as the exact quotient because a
    non-fp16 quotient lies at least 2^-24/(L-1) from every fp16 value, far
    more than the float64 rounding error.  Rows with hi == lo get scale 0.
    """
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    d = hi - lo                                           # exact (float32/fp16 operands)
    q = d / float(L - 1)
    s = q.astype(np.float16)                              # nearest fp16
    # settle the ceiling exactly: fp16 * (L - 1) is exact in float64
    up = s.astype(np.float64) * (L - 1) < d
    s = np.where(up, np.nextafter(s, np.float16(np.inf)), s)
    down = np.nextafter(s, np.float16(-np.inf)).astype(np.float64) * (L - 1) >= d
    s = np.where(down & (q > 0), np.nextafter(s, np.float16(-np.inf)), s)
    s = np.where(q == 0, np.float16(0.0), s)
    return s.astype(np.float16)


def quantize_rows(x: np.ndarray, L: int):
    """Affine L-level quantization of fp16 rows (last axis = 128 values).

    Returns (codes int64[..., 128], scale fp16[...], minimum fp16[...]).
    codes_i = clamp(round_half_even((x_i - min) / scale), 0, L - 1); a row
    whose max equals its min gets scale 0 and all codes 0 (open on the pages).  A
    minimum of -0 is stored as +0 (same arithmetic, one canonical meta byte
    pattern; open on the pages).
    """
    if not (3 <= L <= 65536):
        raise ValueError("L must be in [3, 65536]")
    xh = np.asarray(x, dtype=np.float16)
    if xh.shape[-1] != HEAD_DIM:
        raise ValueError("rows must hold 128 values")
    x64 = xh.astype(np.float64)
    lo = x64.min(axis=-1) + 0.0                           # a zero minimum is stored as +0
    hi = x64.max(axis=-1)
    s16 = scale_fp16_ceil(lo, hi, L)
    s64 = s16.astype(np.float64)
    safe = np.where(s64 > 0, s64, 1.0)
    t = (x64 - lo[..., None]) / safe[..., None]           # numerator exact
    codes = np.rint(t)                                    # ties to even
    codes = np.clip(codes, 0, L - 1)
    codes = np.where((s64 > 0)[..., None], codes, 0.0)
    return codes.astype(np.int64), s16, lo.astype(np.float16)


def hadamard128() -> np.ndarray:
    """Normalized Sylvester Hadamard matrix, float64: H[i, j] =
    (-1)^popcount(i & j) / sqrt(128).  Symmetric, H @ H = I."""
    i = np.arange(HEAD_DIM)
    par = np.zeros((HEAD_DIM, HEAD_DIM), dtype=np.int64)
    for bit in range(7):
        par += ((i[:, None] >> bit) & (i[None, :] >> bit) & 1)
    return np.where(par % 2 == 0, 1.0, -1.0) / math.sqrt(HEAD_DIM)


HADAMARD_SCALE_F32 = np.float32(1.0 / math.sqrt(HEAD_DIM))


def rotate_rows_f32(x: np.ndarray) -> np.ndarray:
    """Hadamard rotation of fp16 rows as the quantizer defines it, float32.

    y = x as float32; for bit = 0 .. 6, every index pair (i, i + 2^bit) with
    that bit clear in i becomes (y_i + y_j, y_i - y_j), each sum and
    difference rounded to float32; finally y * float32(1/sqrt(128)).  Up to
    those roundings this is hadamard128() @ x.  The order of the stages is a
    convention (parity unpinned beyond the rounding bound; see the header).
    """
    y = np.asarray(x, dtype=np.float16).astype(np.float32).copy()
    if y.shape[-1] != HEAD_DIM:
        raise ValueError("rows must hold 128 values")
    for bit in range(7):
        lo_idx = np.array([i for i in range(HEAD_DIM) if not (i >> bit) & 1])
        hi_idx = lo_idx + (1 << bit)
        a = y[..., lo_idx]
        b = y[..., hi_idx]
        y[..., lo_idx] = a + b                            # float32 arithmetic
        y[..., hi_idx] = a - b
    return (y * HADAMARD_SCALE_F32).astype(np.float32)


def fp16_floor(v: np.ndarray) -> np.ndarray:
    """Largest fp16 value <= v (elementwise, |v| within the fp16 range)."""
    v = np.asarray(v, dtype=np.float64)
    h = v.astype(np.float16)                              # nearest
    above = h.astype(np.float64) > v
    h = np.where(above, np.nextafter(h, np.float16(-np.inf)), h)
    return h.astype(np.float16)


def quantize_rows_rotated(x: np.ndarray, L: int):
    """Hadamard-rotated affine quantization of fp16 rows.

    y = rotate_rows_f32(x); min = fp16_floor(min y) (so that every y - min >=
    0 is representable by the codes); scale = smallest fp16 >= (max y -
    min) / (L - 1); codes = clamp(round_half_even((y - min) / scale), 0,
    L - 1), the division and the rounding decided exactly.
    Returns (codes int64[..., 128], scale fp16[...], minimum fp16[...]).
    """
    y = rotate_rows_f32(x).astype(np.float64)             # float32 values, exact in float64
    lo = fp16_floor(y.min(axis=-1)).astype(np.float64) + 0.0
    hi = y.max(axis=-1)
    s16 = scale_fp16_ceil(lo, hi, L)
    s64 = s16.astype(np.float64)
    safe = np.where(s64 > 0, s64, 1.0)
    num = y - lo[..., None]                               # exact: float32 - fp16 in float64
    codes = np.rint(num / safe[..., None])
    # settle near-ties exactly: compare num with (c +/- 1/2) * scale, all exact in float64
    half = (codes + 0.5) * safe[..., None]                # products of <= 17 + 11 bits: exact
    below = (codes - 0.5) * safe[..., None]
    codes = np.where(num > half, codes + 1, codes)
    codes = np.where(num < below, codes - 1, codes)
    tie_up = num == half
    tie_dn = num == below
    codes = np.where(tie_up & (codes % 2 == 1), codes + 1, codes)
    codes = np.where(tie_dn & (codes % 2 == 1), codes - 1, codes)
    codes = np.clip(codes, 0, L - 1)
    codes = np.where((s64 > 0)[..., None], codes, 0.0)
    return codes.astype(np.int64), s16, lo.astype(np.float16)


def dequantize_rows(codes: np.ndarray, scale: np.ndarray, minimum: np.ndarray) -> np.ndarray:
    """x_hat = min + code * scale, float64."""
    return (np.asarray(minimum, dtype=np.float64)[..., None]
            + np.asarray(codes, dtype=np.float64)
            * np.asarray(scale, dtype=np.float64)[..., None])


# --------------------------------------------------------------------------
# Pack (SemKV Table 6 fixes the code-bit rates only: 2.333 bits for 5
# levels = 3 codes per 7 bits, 2.600 for 6 levels; the layout is ours).
# --------------------------------------------------------------------------

_GROUPS = {2: (8, 8), 3: (5, 8), 4: (4, 8), 5: (3, 7), 6: (3, 8),
           8: (1, 3), 16: (2, 8), 65536: (1, 16)}


def group_params(L: int):
    """(g, b): g base-L codes share one b-bit field."""
    if L in _GROUPS:
        return _GROUPS[L]
    return 1, int(math.ceil(math.log2(L)))


def row_bytes(L: int) -> int:
    """Packed bytes of one 128-code row: ceil(ceil(128/g) * b / 8)."""
    g, b = group_params(L)
    nfields = -(-HEAD_DIM // g)
    return -(-nfields * b // 8)


def pack_rows(codes: np.ndarray, L: int) -> np.ndarray:
    """Pack int codes [..., 128] into uint8 [..., row_bytes(L)]."""
    g, b = group_params(L)
    c = np.asarray(codes, dtype=np.int64)
    lead = c.shape[:-1]
    c = c.reshape(-1, HEAD_DIM)
    nfields = -(-HEAD_DIM // g)
    padded = np.zeros((c.shape[0], nfields * g), dtype=np.int64)
    padded[:, :HEAD_DIM] = c
    digits = padded.reshape(c.shape[0], nfields, g)
    weights = np.array([L ** i for i in range(g)], dtype=np.int64)
    fields = (digits * weights).sum(axis=-1)              # first code = lowest digit
    bits = (fields[..., None] >> np.arange(b)) & 1        # LSB first
    bits = bits.reshape(c.shape[0], nfields * b)
    R = row_bytes(L)
    stream = np.zeros((c.shape[0], R * 8), dtype=np.uint8)
    stream[:, :nfields * b] = bits
    out = np.packbits(stream, axis=-1, bitorder="little")
    return out.reshape(lead + (R,))


def unpack_rows(packed: np.ndarray, L: int) -> np.ndarray:
    """Inverse of pack_rows: uint8 [..., row_bytes(L)] -> int64 [..., 128]."""
    g, b = group_params(L)
    p = np.asarray(packed, dtype=np.uint8)
    lead = p.shape[:-1]
    p = p.reshape(-1, p.shape[-1])
    nfields = -(-HEAD_DIM // g)
    bits = np.unpackbits(p, axis=-1, bitorder="little")[:, :nfields * b]
    bits = bits.reshape(p.shape[0], nfields, b).astype(np.int64)
    fields = (bits << np.arange(b)).sum(axis=-1)
    digits = np.stack([(fields // (L ** i)) % L for i in range(g)], axis=-1)
    codes = digits.reshape(p.shape[0], nfields * g)[:, :HEAD_DIM]
    return codes.reshape(lead + (HEAD_DIM,))


def fp16_bits(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float16).view(np.uint16)


# --------------------------------------------------------------------------
# The mixed-precision cache (SemKV Fig. 5: per-token precision broadcast to
# every layer and KV head, applied to keys and values alike).
# --------------------------------------------------------------------------


@dataclass
class Pools:
    """Quantized cache of one batch, in the oracle's own plain layout.

    codes_*  uint8 [B][layers][kv][2][rows][R(L)]   (index 2: 0 = K, 1 = V)
    meta_*   uint16 [B][layers][kv][2][rows][2]      fp16 bits {scale, min}
    tok_*    int32 [B][rows]                         slot -> token index
    """
    L_high: int
    L_low: int
    codes_high: np.ndarray
    meta_high: np.ndarray
    tok_high: np.ndarray
    codes_low: np.ndarray
    meta_low: np.ndarray
    tok_low: np.ndarray
    rotate: bool = False        # rows hold Hadamard-rotated values


def quantize_pack_cache(K: np.ndarray, V: np.ndarray, perm: np.ndarray, k_high: int,
                        L_high: int, L_low: int, token_base: int = 0,
                        rotate: bool = False) -> Pools:
    """Quantize and pack every row of K and V [B][layers][kv][n][128].

    Slot j of the high pool holds token perm[b][j] (j < k_high); slot j of the
    low pool holds token perm[b][k_high + j].  Both K and V of a token use the
    same level count (SemKV Fig. 5).  tok_* records token_base + token.  With
    rotate, rows are quantized by quantize_rows_rotated.
    """
    qrows = quantize_rows_rotated if rotate else quantize_rows
    K = np.asarray(K, dtype=np.float16)
    V = np.asarray(V, dtype=np.float16)
    perm = np.asarray(perm)
    B = K.shape[0]
    kv = np.stack([K, V], axis=3)                         # [B][l][g][2][n][128]
    out = {}
    for name, L, sel in (("high", L_high, perm[:, :k_high]), ("low", L_low, perm[:, k_high:])):
        rows = np.stack([kv[b][:, :, :, sel[b], :] for b in range(B)])   # [B][l][g][2][rows][128]
        codes, s16, m16 = qrows(rows, L)
        out["codes_" + name] = pack_rows(codes, L)
        out["meta_" + name] = np.stack([fp16_bits(s16), fp16_bits(m16)], axis=-1)
        out["tok_" + name] = (sel + token_base).astype(np.int32)
    return Pools(L_high=L_high, L_low=L_low, rotate=rotate, **out)


def dequantize_pool(codes: np.ndarray, meta: np.ndarray, L: int) -> np.ndarray:
    """Packed pool rows -> float64 values [..., rows, 128]."""
    c = unpack_rows(codes, L)
    m = np.asarray(meta, dtype=np.uint16)
    s = m[..., 0].view(np.float16)
    lo = m[..., 1].view(np.float16)
    return dequantize_rows(c, s, lo)


# --------------------------------------------------------------------------
# Decode attention over the mixed cache (SemKV Figs. 1 and 5: the quantized
# cache is what decoding reads; the backbones of Table 2 use grouped-query
# attention, so query head h reads KV head h // (Hq / Hkv)).
# --------------------------------------------------------------------------


def attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray, sm_scale: float) -> np.ndarray:
    """softmax(sm_scale * q . k) weighted sum of v, one query head, float64.

    q [128]; keys, values [T][128].  Summation order is immaterial.
    """
    z = sm_scale * (keys @ np.asarray(q, dtype=np.float64))
    z = z - z.max()
    p = np.exp(z)
    p = p / p.sum()
    return p @ values


def decode_attention(q: np.ndarray, pools: Pools, sm_scale: float, layer0: int = 0,
                     tail_kv: np.ndarray | None = None, n_tail: int = 0) -> np.ndarray:
    """Decode attention for every (b, layer, query head).

    q       fp16 [B][nl][Hq][128], queries for layers layer0 .. layer0+nl-1
    pools   the quantized rows (both pools), all tokens
    tail_kv fp16 [B][layers][kv][2][block][128]; its first n_tail rows are
            the not-yet-quantized newest tokens, read exactly
    returns float64 [B][nl][Hq][128]

    One softmax over every cached token.  With rotated pools the rotation
    belongs to the quantizer: the pool rows hold the quantized H k and H v,
    and as H is orthogonal and symmetric, q . k = (H q) . (H k) and
    sum p v = H (sum p H v).  So their logits take the exactly rotated query
    H q (float64, no rounding: the pages define none) and their share of the
    output is rotated back exactly.  The fp16 tail holds rows that have not
    been quantized, hence not rotated: their logits take the query as given
    and their values enter the output as they are.
    """
    H = hadamard128() if pools.rotate else None
    q_raw = np.asarray(q, dtype=np.float16).astype(np.float64)
    q_pool = q_raw @ H if H is not None else q_raw       # H symmetric: rows -> H q
    B, nl, Hq, _ = q_raw.shape
    Hkv = pools.codes_high.shape[2]
    group = Hq // Hkv
    out = np.zeros(q_raw.shape, dtype=np.float64)
    for b in range(B):
        for li in range(nl):
            layer = layer0 + li
            parts_k, parts_v = [], []
            for codes, meta, L in ((pools.codes_high, pools.meta_high, pools.L_high),
                                   (pools.codes_low, pools.meta_low, pools.L_low)):
                if codes.shape[4] == 0:
                    continue
                x = dequantize_pool(codes[b, layer], meta[b, layer], L)   # [kv][2][rows][128]
                parts_k.append(x[:, 0])
                parts_v.append(x[:, 1])
            kp = np.concatenate(parts_k, axis=1) if parts_k else np.zeros((Hkv, 0, HEAD_DIM))
            vp = np.concatenate(parts_v, axis=1) if parts_v else np.zeros((Hkv, 0, HEAD_DIM))
            if tail_kv is not None and n_tail > 0:
                t = np.asarray(tail_kv[b, layer], dtype=np.float16).astype(np.float64)
                kt, vt = t[:, 0, :n_tail], t[:, 1, :n_tail]
            else:
                kt = vt = np.zeros((Hkv, 0, HEAD_DIM))
            P = kp.shape[1]
            for h in range(Hq):
                g = h // group
                z = sm_scale * np.concatenate([kp[g] @ q_pool[b, li, h], kt[g] @ q_raw[b, li, h]])
                z = z - z.max()
                p = np.exp(z)
                p = p / p.sum()
                o_pool = p[:P] @ vp[g]
                out[b, li, h] = (H @ o_pool if H is not None else o_pool) + p[P:] @ vt[g]
    return out


# --------------------------------------------------------------------------
# Generation-time block-exact quantization (SemKV Fig. 6: scores of new
# tokens accumulate; each completed block is ranked with the same top-r rule
# and quantized; the newest partial block stays fp16 while decoding; at the
# end of a turn the residual block is quantized with the same rule).
# --------------------------------------------------------------------------


@dataclass
class GenerationCache:
    """Streaming oracle of the prompt + generation path of one batch."""
    layers: int
    kv_heads: int
    L_high: int
    L_low: int
    r: float
    block: int = 128
    batch: int = 1
    pools: Pools | None = None
    tail_k: list = field(default_factory=list)   # list of [B][layers][kv][128] fp16
    tail_v: list = field(default_factory=list)
    tail_s: list = field(default_factory=list)   # list of [B] fp32
    n_tokens: int = 0
    rotate: bool = False                         # Hadamard-rotated pools (the tail stays fp16)

    def _empty_pools(self) -> Pools:
        B, l, g = self.batch, self.layers, self.kv_heads
        def z(L):
            return (np.zeros((B, l, g, 2, 0, row_bytes(L)), np.uint8),
                    np.zeros((B, l, g, 2, 0, 2), np.uint16), np.zeros((B, 0), np.int32))
        ch, mh, th = z(self.L_high)
        cl, ml, tl = z(self.L_low)
        return Pools(self.L_high, self.L_low, ch, mh, th, cl, ml, tl, rotate=self.rotate)

    def _append_pools(self, new: Pools):
        if self.pools is None:
            self.pools = self._empty_pools()
        p = self.pools
        self.pools = Pools(
            self.L_high, self.L_low,
            np.concatenate([p.codes_high, new.codes_high], axis=4),
            np.concatenate([p.meta_high, new.meta_high], axis=4),
            np.concatenate([p.tok_high, new.tok_high], axis=1),
            np.concatenate([p.codes_low, new.codes_low], axis=4),
            np.concatenate([p.meta_low, new.meta_low], axis=4),
            np.concatenate([p.tok_low, new.tok_low], axis=1),
            rotate=self.rotate)

    def prompt(self, K, V, scores):
        """Quantize a whole prompt with one global top-r over its scores."""
        n = K.shape[3]
        k = topr_count(n, self.r)
        perm, _ = rank_topr_batch(scores, k)
        self._append_pools(quantize_pack_cache(K, V, perm, k, self.L_high, self.L_low,
                                               token_base=self.n_tokens, rotate=self.rotate))
        self.n_tokens += n

    def _quantize_tail(self):
        nt = len(self.tail_k)
        if nt == 0:
            return
        K = np.stack(self.tail_k, axis=3)        # [B][layers][kv][nt][128]
        V = np.stack(self.tail_v, axis=3)
        s = np.stack(self.tail_s, axis=1)        # [B][nt]
        k = topr_count(nt, self.r)
        perm, _ = rank_topr_batch(s, k)
        self._append_pools(quantize_pack_cache(K, V, perm, k, self.L_high, self.L_low,
                                               token_base=self.n_tokens - nt, rotate=self.rotate))
        self.tail_k, self.tail_v, self.tail_s = [], [], []

    def append(self, k_new, v_new, score_new):
        """Append one generated token ([B][layers][kv][128] K and V, [B] score)."""
        self.tail_k.append(np.asarray(k_new, dtype=np.float16))
        self.tail_v.append(np.asarray(v_new, dtype=np.float16))
        self.tail_s.append(np.asarray(score_new, dtype=np.float32))
        self.n_tokens += 1
        if len(self.tail_k) == self.block:
            self._quantize_tail()

    def flush(self):
        """End of turn: quantize the residual block with the same top-r rule."""
        self._quantize_tail()

    @property
    def n_tail(self) -> int:
        return len(self.tail_k)

    def tail_array(self) -> np.ndarray:
        """Tail as fp16 [B][layers][kv][2][block][128] (rows past n_tail are 0)."""
        B = self.batch
        t = np.zeros((B, self.layers, self.kv_heads, 2, self.block, HEAD_DIM), np.float16)
        for i, (kk, vv) in enumerate(zip(self.tail_k, self.tail_v)):
            t[:, :, :, 0, i] = kk
            t[:, :, :, 1, i] = vv
        return t

    def decode(self, q, sm_scale, layer0=0):
        pools = self.pools if self.pools is not None else self._empty_pools()
        return decode_attention(q, pools, sm_scale, layer0=layer0,
                                tail_kv=self.tail_array(), n_tail=self.n_tail)


# --------------------------------------------------------------------------
# Ragged batches (SemKV Fig. 6: each prompt is ranked and quantized on its
# own and each sequence's generation blocks fill at their own pace; SemKV
# Table 2: multi-turn use, with the residual block quantized at every turn's
# end).  Reading: the sequences of a batch share nothing but the buffers, so
# a ragged batch is its sequences taken one at a time -- one batch-of-one
# GenerationCache per sequence, driven by that sequence's own events.
# --------------------------------------------------------------------------


class RaggedGeneration:
    """Streaming oracle of a batch whose sequences advance independently."""

    def __init__(self, batch, layers, kv_heads, L_high, L_low, r, block=128, rotate=False):
        self.seqs = [GenerationCache(layers=layers, kv_heads=kv_heads, L_high=L_high,
                                     L_low=L_low, r=r, block=block, batch=1, rotate=rotate)
                     for _ in range(batch)]

    def prompt(self, b, K, V, scores):
        """Prompt of sequence b: K, V [layers][kv][n][128] fp16, scores [n].
        A prompt starts a turn, so the sequence's tail must be empty."""
        g = self.seqs[b]
        if g.n_tail != 0:
            raise ValueError("a prompt needs an empty tail (flush the previous turn first)")
        g.prompt(np.asarray(K)[None], np.asarray(V)[None], np.asarray(scores, np.float32)[None])

    def append(self, b, k_new, v_new, score):
        """One generated token of sequence b: k_new, v_new [layers][kv][128]."""
        self.seqs[b].append(np.asarray(k_new)[None], np.asarray(v_new)[None],
                            np.asarray([score], np.float32))

    def flush(self, b):
        self.seqs[b].flush()

    def counters(self, b):
        """(n_high, n_low, n_tail, n_tokens) of sequence b."""
        g = self.seqs[b]
        p = g.pools
        nh = 0 if p is None else p.codes_high.shape[4]
        nl = 0 if p is None else p.codes_low.shape[4]
        return nh, nl, g.n_tail, g.n_tokens

    def pools(self, b) -> Pools:
        g = self.seqs[b]
        return g.pools if g.pools is not None else g._empty_pools()

    def tail_array(self, b):
        return self.seqs[b].tail_array()[0]

    def decode(self, b, q, sm_scale, layer0=0):
        """q [nl][Hq][128] of sequence b -> [nl][Hq][128]."""
        return self.seqs[b].decode(np.asarray(q)[None], sm_scale, layer0=layer0)[0]


# --------------------------------------------------------------------------
# Storage accounting (SemKV Tables 3-6, Fig. 11).
# --------------------------------------------------------------------------


def nominal_bits(k: int, n: int, L_high: int, L_low: int) -> float:
    """Average code bits on the level grid: (k log2 Lh + (n-k) log2 Ll) / n."""
    return (k * math.log2(L_high) + (n - k) * math.log2(L_low)) / n


def format_bits(k: int, n: int, L_high: int, L_low: int, meta_bytes: int = 4) -> float:
    """Stored bits per value of this format: packed row bytes + 4 meta bytes."""
    per_row = k * (row_bytes(L_high) + meta_bytes) + (n - k) * (row_bytes(L_low) + meta_bytes)
    return per_row * 8.0 / (HEAD_DIM * n)
