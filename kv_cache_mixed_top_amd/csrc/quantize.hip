// Quantize and pack K/V rows into the two precision pools (SemKV page,
// Fig. 5: one precision per token, applied to K and V of every layer and KV
// head; Table 6: affine integer-level quantizer with two fp16 scalars per
// 128-value row).
//
// Workgroup = 256 threads = 64 rows x 4 lanes; one workgroup writes 64
// consecutive slots of one pool plane (sequence, layer, KV head, K|V).  Lane
// q of a row loads the 16-byte pieces at byte offsets 16q + 64i (i = 0..3),
// so each load instruction of a quad covers 64 contiguous bytes.
//
// Codes: c = round-half-even((x - m) / s).  The fast path (pools of 3, 4, 5,
// 6, 8 and 16 levels) evaluates y = (x - m)/s + D (D a small even integer)
// as one fp32 FMA with fl(1/s) and converts it to a byte; a group of 8 values
// with one near a half-integer (within the bound of that evaluation's error)
// is re-read and settled exactly in double with the residuals
// x - m - (c0 +/- 1/2) s.  The generic path (any level count) evaluates
// y = (x - m) * fl(1/s) and settles each value near a half-integer the same
// way.
//
// Packing: codes go to LDS; each output byte is assembled from the fields
// that overlap it.  K planes hold rows back to back; V planes are byte-planar
// in 16-row tiles (the layout the decode kernel reads 8 tokens' byte from).
// Bytes of a dword shared with rows of another workgroup are stored one by
// one.
#include <type_traits>

#include "semkv_internal.h"

namespace semkv {
namespace {

constexpr int kRows = 64;
constexpr int kThreads = 256;
constexpr int kCodeStride = kHeadDim + 2;   // u16 codes per LDS row (pad)

// Exact round-half-even of (x - m)/s given a candidate c0 within 1 of it.
__device__ __forceinline__ float exact_code(float x, float m, float s, float c0) {
  // exact for fp16 x; a rotated fp32 x rounds only when |x| << |m|, by less
  // than the spacing of m + (c +/- 1/2) s, so the signs below still hold
  const double d = (double)x - (double)m;
  const double sd = (double)s;
  const double c = (double)c0;
  const double e_hi = d - (c + 0.5) * sd;           // exact (<= 45 significant bits)
  const double e_lo = d - (c - 0.5) * sd;
  const bool odd = (((int)c0) & 1) != 0;
  if (e_hi > 0.0) return c0 + 1.0f;
  if (e_hi == 0.0) return odd ? c0 + 1.0f : c0;
  if (e_lo < 0.0) return c0 - 1.0f;
  if (e_lo == 0.0) return odd ? c0 - 1.0f : c0;
  return c0;
}

// Exchange with lane ^ 1 / lane ^ 2 inside each quad (DPP quad permutes).
__device__ __forceinline__ float quad_xor1(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
}

// Hadamard rotation of one row held by a quad (normalized Sylvester H_128,
// fp32), the lane holding dims 8q + 32i + e as v[8i + e]: butterflies on the
// index bits 0 .. 6 in order -- bits 0-2 (e) and 5-6 (i) within the lane,
// bits 3-4 (q) across the quad -- each pair (a, b) -> (a + b, a - b), then
// one multiply by fp32(1/sqrt(128)).  kFrom: the first within-lane bit still
// to do (1 when the caller has done bit 0 already); kScale = false leaves the
// multiply to the caller.
//
// Across the quad each value takes one v_fmac_f32 with a DPP source: own +
// b * partner, b = +1 in the lower lane and -1 in the upper one.  The upper
// lane so gets hi - lo, the exact negation of lo - hi (round to nearest is
// symmetric), and keeps it: after both stages the lane holds its values times
// sigma = (-1)^(q0 + q1), and the within-lane stages keep that sign.  The
// function returns sigma; with kScale the multiply takes it out.
constexpr float kRotScale = 0.08838834764831845f;          // fp32(1/sqrt(128))

// x += b * (x of lane ^ 1), resp. lane ^ 2, within the quad.  The s_nop gives
// the two wait states a DPP read needs after a VALU write of its source; the
// caller puts a scheduling barrier before the first of a run of these, so
// that the compiler places no write of a later source between them.
template <int kM, bool kFirst>
__device__ __forceinline__ void quad_fmac(float& x, float b) {
  if constexpr (kM == 1) {
    if constexpr (kFirst)
      asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %0, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
                   : "+v"(x) : "v"(b));
    else
      asm volatile("v_fmac_f32_dpp %0, %0, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf" : "+v"(x) : "v"(b));
  } else {
    if constexpr (kFirst)
      asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %0, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
                   : "+v"(x) : "v"(b));
    else
      asm volatile("v_fmac_f32_dpp %0, %0, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf" : "+v"(x) : "v"(b));
  }
}

template <int kFrom = 0, bool kScale = true>
__device__ __forceinline__ float rotate_row(float (&v)[32], int q) {
#pragma unroll
  for (int bit = kFrom; bit < 3; ++bit)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!((e >> bit) & 1)) {
          const float x0 = v[8 * i + e], x1 = v[8 * i + e + (1 << bit)];
          v[8 * i + e] = x0 + x1;
          v[8 * i + e + (1 << bit)] = x0 - x1;
        }
  // bits 3, 4: lane q ^ 1, then q ^ 2
  const float b1 = (q & 1) ? -1.0f : 1.0f, b2 = (q & 2) ? -1.0f : 1.0f;
  __builtin_amdgcn_sched_barrier(0);
  quad_fmac<1, true>(v[0], b1);
#pragma unroll
  for (int j = 1; j < 32; ++j) quad_fmac<1, false>(v[j], b1);
  quad_fmac<2, true>(v[0], b2);
#pragma unroll
  for (int j = 1; j < 32; ++j) quad_fmac<2, false>(v[j], b2);
  __builtin_amdgcn_sched_barrier(0);
  const float sigma = b1 * b2;
#pragma unroll
  for (int bit = 0; bit < 2; ++bit)                        // bits 5, 6: i ^ (1 << bit)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (!((i >> bit) & 1))
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x0 = v[8 * i + e], x1 = v[8 * (i + (1 << bit)) + e];
          v[8 * i + e] = x0 + x1;
          v[8 * (i + (1 << bit)) + e] = x0 - x1;
        }
  if constexpr (kScale) {
    const float k = sigma * kRotScale;
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] *= k;
  }
  return kScale ? 1.0f : sigma;
}

// What one workgroup's pool writes: its row count, where its rows start in
// perm, its first destination slot and the token index base.  A ragged batch
// takes them from the sequence's device counters; a sequence whose rows would
// not fit (or, for a prompt, whose tail is not empty) writes nothing, and the
// counter update that follows records that in its status word.  (kRagged
// is a compile-time choice, so that the kernels of uniform batches carry
// none of the ragged bookkeeping.)
struct PoolPart {
  int count, perm_off;
  int64_t start, token_base, perm_ld;
};
template <bool kRagged>
__device__ __forceinline__ PoolPart pool_part(const QuantArgs& a, int pool, int b) {
  PoolPart pp;
  if constexpr (!kRagged) {
    pp.count = pool == 0 ? a.k_high : a.n - a.k_high;
    pp.perm_off = pool == 0 ? 0 : a.k_high;
    pp.start = a.start[pool];
    pp.token_base = a.token_base;
    pp.perm_ld = a.n;
    return pp;
  }
  const int64_t* sq = a.seq + (int64_t)b * kSeqWords;
  const int n = a.n_seq[b];
  const int k = (int)topr_count(n, a.r);
  const bool skip = (a.tail_mode == 0 && sq[kSeqTail] != 0) || sq[kSeqHigh] + k > a.cap[0] ||
                    sq[kSeqLow] + (n - k) > a.cap[1];
  pp.count = skip ? 0 : (pool == 0 ? k : n - k);
  pp.perm_off = pool == 0 ? 0 : k;
  pp.start = sq[pool == 0 ? kSeqHigh : kSeqLow];
  pp.token_base = sq[kSeqTokens] - sq[kSeqTail];
  pp.perm_ld = a.ld_perm;
  return pp;
}

// One 64-slot tile of one pool plane.  LF = level count known at compile
// time (6 or 5), or 0 for the runtime format of the pool.
template <int LF, bool kRot>
__device__ __forceinline__ void quantize_tile(const QuantArgs& a, const PoolPart& pp, int pool,
                                              int tile_in_pool, uint16_t* codes) {
  const RowFmt f = LF ? row_fmt(LF) : a.fmt[pool];
  const int count = pp.count;
  const int perm_off = pp.perm_off;
  const int y = blockIdx.y;
  const int kvsel = y & 1;
  const int head = (y >> 1) % a.kv_heads;
  const int layer = (y >> 1) / a.kv_heads;
  const int b = blockIdx.z;
  const int row0 = tile_in_pool * kRows;
  const int nrows = min(kRows, count - row0);

  const int tid = threadIdx.x;
  const int r = tid >> 2, q = tid & 3;
  const bool valid = r < nrows;
  const int64_t plane = (((int64_t)b * a.layers + layer) * a.kv_heads + head) * 2 + kvsel;
  const int64_t slot0 = pp.start + row0;

  // ---- load 32 values of this row (d = 8q + 32i + e)
  int token = 0;
  float v[32];
  if (valid) {
    token = a.perm[(int64_t)b * pp.perm_ld + perm_off + row0 + r];
    const uint16_t* src = a.src[kvsel] + (int64_t)b * a.sb + (int64_t)layer * a.sl +
                          (int64_t)head * a.sh + (int64_t)token * a.st;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 w = *reinterpret_cast<const uint4*>(src + 8 * q + 32 * i);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * i + 2 * e] = h2f((uint16_t)(ws[e] & 0xFFFFu));
        v[8 * i + 2 * e + 1] = h2f((uint16_t)(ws[e] >> 16));
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.f;
  }

  // ---- optional Hadamard rotation of the row
  if constexpr (kRot) rotate_row(v, q);

  // ---- row min / max over the quad
  float lo = v[0], hi = v[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) {
    lo = fminf(lo, v[i]);
    hi = fmaxf(hi, v[i]);
  }
  lo = fminf(lo, __shfl_xor(lo, 1, 64));
  lo = fminf(lo, __shfl_xor(lo, 2, 64));
  hi = fmaxf(hi, __shfl_xor(hi, 1, 64));
  hi = fmaxf(hi, __shfl_xor(hi, 2, 64));
  if constexpr (kRot) lo = fp16_floor(lo);   // rotated values are fp32: the stored minimum is fp16
  lo = lo + 0.0f;   // a zero minimum is stored as +0

  const uint16_t sbits = scale_ceil_bits(lo, hi, f.L);
  const float s = h2f(sbits);
  const float lmax = (float)(f.L - 1);

  // ---- codes
  uint16_t* crow = codes + r * kCodeStride;
  if (s > 0.0f) {
    const float rs = 1.0f / s;
    const float eps = lmax * 0x1p-20f + 0x1p-22f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = v[8 * i + e];
        const float yv = (x - lo) * rs;
        float c = rintf(yv);
        if (fabsf(fabsf(yv - c) - 0.5f) <= eps) c = exact_code(x, lo, s, c);
        c = fminf(fmaxf(c, 0.0f), lmax);
        crow[8 * q + 32 * i + e] = (uint16_t)(int)c;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) crow[8 * q + 32 * i + e] = 0;
  }

  if (valid && q == 0) {
    const int64_t slot = slot0 + r;
    a.meta[pool][plane * a.cap[pool] + slot] = (uint32_t)sbits | ((uint32_t)f2h(lo) << 16);
    if (layer == 0 && head == 0 && kvsel == 0)
      a.tok[pool][(int64_t)b * a.cap[pool] + slot] = (int32_t)(pp.token_base + token);
  }
  __syncthreads();

  // ---- pack.  K planes: rows back to back.  V planes: byte-planar in
  // 16-row tiles (byte j of row r at (r/16)*16R + 16j + r%16).  Each output
  // byte is assembled from the fields overlapping it; bytes of rows outside
  // this workgroup's slots are left untouched.
  const int R = f.R;
  uint8_t* base = a.codes[pool] + plane * a.cap[pool] * R;
  const int64_t s_lo = slot0, s_hi = slot0 + nrows;
  int64_t B0, B1;
  if (kvsel == 0) {
    B0 = s_lo * R;
    B1 = s_hi * R;
  } else {
    B0 = (s_lo >> 4) * 16 * R;
    B1 = ((s_hi + 15) >> 4) * 16 * R;
  }
  const int64_t w0 = B0 >> 2, w1 = (B1 + 3) >> 2;
  const int nfields = (kHeadDim + f.g - 1) / f.g;
  uint32_t pw[6];
  pw[0] = 1;
#pragma unroll
  for (int i = 1; i < 6; ++i) pw[i] = pw[i - 1] * (uint32_t)f.L;
  const uint32_t fmask = (1u << f.b) - 1u;

  for (int64_t w = w0 + tid; w < w1; w += kThreads) {
    uint32_t val = 0, inmask = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t pbyte = 4 * w + e;
      if (pbyte < B0 || pbyte >= B1) continue;
      int64_t row_abs;
      int jb;
      if (kvsel == 0) {
        row_abs = pbyte / R;
        jb = (int)(pbyte - row_abs * R);
      } else {
        const int64_t tile = pbyte / (16 * R);
        const int rem = (int)(pbyte - tile * 16 * R);
        jb = rem >> 4;
        row_abs = tile * 16 + (rem & 15);
      }
      const int64_t row = row_abs - s_lo;
      if (row < 0 || row >= nrows) continue;
      inmask |= 1u << e;
      const int bit0 = 8 * jb;
      const int fl = bit0 / f.b;
      const int fh = min((bit0 + 7) / f.b, nfields - 1);
      uint32_t byte = 0;
      for (int fi = fl; fi <= fh; ++fi) {
        uint32_t fv = 0;
        for (int i = 0; i < f.g; ++i) {
          const int pos = f.g * fi + i;
          if (pos < kHeadDim) fv += (uint32_t)codes[row * kCodeStride + pos] * pw[i];
        }
        fv &= fmask;
        const int shift = f.b * fi - bit0;
        byte |= shift >= 0 ? (fv << shift) : (fv >> (-shift));
      }
      val |= (byte & 0xFFu) << (8 * e);
    }
    if (inmask == 0xFu) {
      reinterpret_cast<uint32_t*>(base)[w] = val;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (inmask & (1u << e)) base[4 * w + e] = (uint8_t)(val >> (8 * e));
    }
  }
}

// ---- fast path for pools of 3, 4, 5, 6, 8 and 16 levels when the tile's
// first slot is a multiple of 16 (every tile of a prompt): the tile's packed
// bytes form one contiguous, 16-byte aligned range of the plane in both
// layouts, which is assembled in LDS and stored with 16-byte writes.
constexpr int kCode8Stride = 136;                 // u8 codes per LDS row: 128 + 8 zero pad
constexpr int kCode8Bytes = kRows * kCode8Stride + 16;
constexpr int kImgBytes = kRows * 64;             // largest packed tile (16 levels)

// packed row bytes of the level counts with a fast path (the row format of
// semkv_common.h: ceil(128 / g) fields of b bits)
template <int L> constexpr int fast_row_bytes() {
  return L == 3 ? 26 : L == 4 ? 32 : L == 5 ? 38 : L == 6 ? 43 : L == 8 ? 48 : 64;
}
__host__ __device__ constexpr bool fast_quant_level(int L) {
  return L == 3 || L == 4 || L == 5 || L == 6 || L == 8 || L == 16;
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The packed image is written once and not read back by this pass: its
// stores are non-temporal.  (Non-temporal loads of the fp16 rows, which are
// read in permuted order, measured slower.)
__device__ __forceinline__ void store_stream(uint4* p, uint4 v) {
  __builtin_nontemporal_store((u32x4){v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

// Smallest fp16 >= (hi - lo) / (L - 1) without a division: the fp32 quotient
// is within 2^-22 of the exact one, so its nearest fp16 is the ceiling or
// the fp16 just below it; s * (L - 1) >= hi - lo is then decided exactly in
// double (an fp16 times an integer below 2^16 and a difference of two fp16).
template <int L>
__device__ __forceinline__ uint16_t scale_ceil_fast(float lo, float hi) {
  const double d = (double)hi - (double)lo;
  if (!(d > 0.0)) return 0;
  uint16_t h = f2h((float)d * (1.0f / (float)(L - 1)));
  if ((double)h2f(h) * (double)(L - 1) < d) ++h;
  return h;
}


// kRot: the rows are Hadamard-rotated (fp32 values kept in registers).
template <int L, bool kRot>
__device__ __forceinline__ void quantize_tile_fast(const QuantArgs& a, const PoolPart& pp, int pool,
                                                   int tile_in_pool, uint8_t* codes8, uint8_t* img) {
  constexpr int R = fast_row_bytes<L>();
  const int count = pp.count;
  const int perm_off = pp.perm_off;
  const int y = blockIdx.y;
  const int kvsel = y & 1;
  const int head = (y >> 1) % a.kv_heads;
  const int layer = (y >> 1) / a.kv_heads;
  const int b = blockIdx.z;
  const int row0 = tile_in_pool * kRows;
  const int nrows = min(kRows, count - row0);
  const int tid = threadIdx.x;
  const int r = tid >> 2, q = tid & 3;
  const bool valid = r < nrows;
  const int64_t plane = (((int64_t)b * a.layers + layer) * a.kv_heads + head) * 2 + kvsel;
  const int64_t slot0 = pp.start + row0;

  // ---- 32 values of this row as 16 fp16 pairs (dims 8q + 32i + 2e + {0,1})
  int token = 0;
  half2_t v[16];
  const uint16_t* src = nullptr;
  if (valid) {
    token = a.perm[(int64_t)b * pp.perm_ld + perm_off + row0 + r];
    src = a.src[kvsel] + (int64_t)b * a.sb + (int64_t)layer * a.sl + (int64_t)head * a.sh +
          (int64_t)token * a.st;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 w = *reinterpret_cast<const uint4*>(src + 8 * q + 32 * i);
      v[4 * i + 0] = __builtin_bit_cast(half2_t, w.x);
      v[4 * i + 1] = __builtin_bit_cast(half2_t, w.y);
      v[4 * i + 2] = __builtin_bit_cast(half2_t, w.z);
      v[4 * i + 3] = __builtin_bit_cast(half2_t, w.w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = (half2_t){0, 0};
  }

  // ---- row min / max: packed fp16 (exact), then the quad; rotated rows:
  // fp32 values, the stored minimum rounded down to fp16
  float yr[kRot ? 32 : 1];
  float rsig = 1.0f;   // rotated rows: yr holds rsig times the sums
  float lo, hi;
  if constexpr (kRot) {
    // bit 0 pairs are the two halves of one fp16 pair: a mixed-precision
    // fma takes them straight from fp16 (exact product, one rounding).  The
    // multiplier 1 is hidden from the optimizer, which would otherwise turn
    // the fma into two conversions and an add.
    float one = 1.0f;
    asm volatile("" : "+v"(one));
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      yr[2 * k & (kRot ? 31 : 0)] = fmaf((float)v[k][1], one, (float)v[k][0]);
      yr[(2 * k + 1) & (kRot ? 31 : 0)] = fmaf((float)v[k][1], -one, (float)v[k][0]);
    }
    // the sums u before the scaling: the rotated value is x = fl(u k), and
    // as rounding is monotone the extremes are fl(min u k), fl(max u k)
    rsig = rotate_row<1, false>(yr, q);   // yr holds rsig u
    lo = yr[0];
    hi = yr[0];
#pragma unroll
    for (int k = 1; k < 32; ++k) {
      lo = fminf(lo, yr[k]);
      hi = fmaxf(hi, yr[k]);
    }
    if (rsig < 0.0f) {
      const float t = lo;
      lo = -hi;
      hi = -t;
    }
    lo *= kRotScale;
    hi *= kRotScale;
  } else {
    half2_t mn = v[0], mx = v[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      mn = __builtin_elementwise_minimum(mn, v[i]);
      mx = __builtin_elementwise_maximum(mx, v[i]);
    }
    lo = fminf((float)mn[0], (float)mn[1]);
    hi = fmaxf((float)mx[0], (float)mx[1]);
  }
  lo = fminf(lo, quad_xor1(lo));
  lo = fminf(lo, quad_xor2(lo));
  hi = fmaxf(hi, quad_xor1(hi));
  hi = fmaxf(hi, quad_xor2(hi));
  if constexpr (kRot) lo = fp16_floor(lo);
  lo = lo + 0.0f;   // a zero minimum is stored as +0

  const uint16_t sbits = scale_ceil_fast<L>(lo, hi);
  const float s = h2f(sbits);

  // ---- codes: y = x * r - m * r in one fma from the fp16 value, r = v_rcp(s)
  // (within 1 ulp).  |y - (x - m)/s| <= 2^-23 (1.5 (L-1) + |m|/s) (1 + 2^-20);
  // a code whose y lies within 2^-22 ((L-1) + |m| r) of a half-integer is
  // settled exactly.  v_cvt_pk_u8_f32 rounds to nearest even and clamps to
  // [0, 255], which is the code elsewhere.  Rotated rows take y = u fl(r k)
  // - m r from the unscaled sum u; against x = fl(u k) that adds at most
  // 2^-23 |x|/s (1 + 2^-22) <= 2^-23 ((L-1) + |m|/s) (1 + 2^-22), so their
  // window is 2^-22 (1.5 (L-1) + 1.25 |m| r).  The settling itself starts
  // from round((x - m) r) with x - m rounded once in fp32 (code error
  // <= 2^-22 (L-1)), which is within 1 of the exact code whatever |m|/s.
  //
  // The fast pass computes y + D instead (D = 10 up to 6 levels, 18 for 8,
  // 34 for 16: an even integer that keeps every y + D inside one binade,
  // [8, 16), [16, 32) or [32, 64)), where the fraction is the low FB = 20,
  // 19 or 18 mantissa bits: the distance of the fraction from 1/2 is then one
  // shift-and-add of the bits and an unsigned minimum, and the packed bytes
  // are code + D (D is even, so ties round alike).  Its error bound grows by
  // the two roundings at that magnitude; the window below is twice the one
  // above plus 2^-FB.  The LDS code array keeps code + D (pads and constant
  // rows too); the field sums take the offset back out in the dot product's
  // accumulator.
  // A constant row (s = 0; also the rows past the tile's end, read as
  // zeros) is coded with scale 1: every value equals m, so y = D exactly
  // and every code is 0, with no branch.
  constexpr int kD = L <= 6 ? 10 : L == 8 ? 18 : 34;
  constexpr int kFB = L <= 6 ? 20 : L == 8 ? 19 : 18;
  constexpr int kSh = 32 - kFB;
  constexpr uint32_t kZeroCode = 0x01010101u * (uint32_t)kD;   // code 0 in four code bytes
  const float sq = s > 0.0f ? s : 1.0f;
  uint32_t cw[8];
  const float rs = __builtin_amdgcn_rcpf(sq);
  const float eps = kRot ? 0x1p-22f * (1.5f * (float)(L - 1) + 1.25f * fabsf(lo) * rs) + 0x1p-30f
                         : 0x1p-22f * ((float)(L - 1) + fabsf(lo) * rs) + 0x1p-30f;
  const float rsk = kRot ? rs * kRotScale : rs;
  const float rsks = kRot ? rsig * rsk : rs;   // y from rsig u: the sign cancels exactly
  const float nb10 = fmaf(-lo, rs, (float)kD);
  constexpr float kUnit = (float)(1u << kFB);
  const float win = (2.0f * eps + 1.0f / kUnit) * kUnit;        // in units of 2^-FB
  const bool wide = !(win < kUnit / 8.0f);                      // then every code is settled
  const uint32_t E = wide ? (1u << (kFB - 3)) : (uint32_t)win + 1u;
  const uint32_t bias = (E - (1u << (kFB - 1))) << kSh;   // (frac - 1/2 + E) mod 2^FB, in the top bits
  const uint32_t thr = (2u * E) << kSh;
  uint32_t umin[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};   // per 8 values
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const float y = fmaf(kRot ? yr[k & (kRot ? 31 : 0)] : (float)v[k >> 1][k & 1], rsks, nb10);
    umin[k >> 3] = min(umin[k >> 3], (__builtin_bit_cast(uint32_t, y) << kSh) + bias);
    cw[k >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(y, k & 3, (k & 3) ? cw[k >> 2] : 0u);
  }
  // dims 8q + 32i .. +8 -> row r of the LDS code array; lane 0 of the quad
  // clears the 8 pad bytes (fields read up to code 131)
  uint8_t* crow = codes8 + r * kCode8Stride;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<uint2*>(crow + 8 * q + 32 * i) = make_uint2(cw[2 * i], cw[2 * i + 1]);
  uint32_t flag = 0u;   // groups of 8 values with a value near a half-integer
#pragma unroll
  for (int i = 0; i < 4; ++i) flag |= (uint32_t)(wide || umin[i] <= thr) << i;
  if (kRot && flag) {
    // rotated rows: the values are still in registers
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!((flag >> i) & 1u)) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float u = rsig * yr[(8 * i + e) & (kRot ? 31 : 0)];
        const float y = fmaf(u, rsk, nb10);
        if (wide || (__builtin_bit_cast(uint32_t, y) << kSh) + bias <= thr) {
          const float x = u * kRotScale;
          const float c = exact_code(x, lo, sq, rintf((x - lo) * rs));
          crow[8 * q + 32 * i + e] = (uint8_t)((int)c + kD);
        }
      }
    }
  } else if (flag) {
    // Rare per group: one of its values lies near a half-integer (with fp16
    // data nearly always an exact tie).  The group's 8 values are read
    // again, and those near a half-integer are settled exactly and their
    // code bytes rewritten; the loop holds few registers.
#pragma unroll 1
    for (int i = 0; i < 4; ++i) {
      if (!((flag >> i) & 1u)) continue;
      const uint4 w = *reinterpret_cast<const uint4*>(src + 8 * q + 32 * i);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = h2f((uint16_t)(ws[e >> 1] >> (16 * (e & 1))));
        const float y = fmaf(x, rs, nb10);
        if (wide || (__builtin_bit_cast(uint32_t, y) << kSh) + bias <= thr) {
          const float c = exact_code(x, lo, sq, rintf((x - lo) * rs));
          crow[8 * q + 32 * i + e] = (uint8_t)((int)c + kD);
        }
      }
    }
  }
  if (q == 0) *reinterpret_cast<uint2*>(crow + 128) = make_uint2(kZeroCode, kZeroCode);
  if (tid < 4) reinterpret_cast<uint32_t*>(codes8 + kRows * kCode8Stride)[tid] = kZeroCode;

  if (valid && q == 0) {
    const int64_t slot = slot0 + r;
    a.meta[pool][plane * a.cap[pool] + slot] = (uint32_t)sbits | ((uint32_t)f2h(lo) << 16);
    if (layer == 0 && head == 0 && kvsel == 0)
      a.tok[pool][(int64_t)b * a.cap[pool] + slot] = (int32_t)(pp.token_base + token);
  }
  __syncthreads();

  // ---- fields (sum_i code[g j + i] L^i, udot4 over the code bytes) -> the
  // tile's byte image: K rows back to back, V byte-planar in 16-row tiles.
  // The layout is uniform per workgroup, so each is its own code path: byte
  // j of this thread's row lands at rowimg + j * kStep.
  auto pack = [&](auto planar_c) {
    constexpr bool kPlanar = decltype(planar_c)::value;
    constexpr int kStep = kPlanar ? 16 : 1;
    uint8_t* rowimg = kPlanar ? img + (r >> 4) * 16 * R + (r & 15) : img + r * R;
    const uint8_t* crow8 = codes8 + r * kCode8Stride;
    if (L == 6) {
      constexpr uint32_t W = 0x00240601u;              // bytes {1, 6, 36, 0}
      constexpr uint32_t Z = 0u - (uint32_t)kD * 43u;  // removes the +D of three codes
#pragma unroll
      for (int u = q; u < 11; u += 4) {                // fields 4u .. 4u+3 of this thread's row
        const uint32_t* c = reinterpret_cast<const uint32_t*>(crow8 + 12 * u);
        const uint32_t c0 = c[0], c1 = c[1], c2 = c[2];
        uint8_t* o = rowimg + 4 * u * kStep;
        o[0] = (uint8_t)__builtin_amdgcn_udot4(c0, W, Z, false);
        o[kStep] = (uint8_t)__builtin_amdgcn_udot4(__builtin_amdgcn_alignbyte(c1, c0, 3), W, Z, false);
        o[2 * kStep] = (uint8_t)__builtin_amdgcn_udot4(__builtin_amdgcn_alignbyte(c2, c1, 2), W, Z, false);
        if (u < 10) o[3 * kStep] = (uint8_t)__builtin_amdgcn_udot4(c2 >> 8, W, Z, false);
      }
    } else if (L == 4) {
      constexpr uint32_t W = 0x40100401u;              // bytes {1, 4, 16, 64}
      constexpr uint32_t Z = 0u - (uint32_t)kD * 85u;
      const uint32_t* c = reinterpret_cast<const uint32_t*>(crow8);
#pragma unroll
      for (int u = q; u < 32; u += 4)                  // byte u = codes 4u .. 4u+3
        rowimg[u * kStep] = (uint8_t)__builtin_amdgcn_udot4(c[u], W, Z, false);
    } else if (L == 16) {
      constexpr uint32_t W = 0x00001001u;              // bytes {1, 16, 0, 0}
      constexpr uint32_t Z = 0u - (uint32_t)kD * 17u;
      const uint32_t* c = reinterpret_cast<const uint32_t*>(crow8);
#pragma unroll
      for (int u = q; u < 32; u += 4) {                // bytes 2u, 2u+1 = codes 4u .. 4u+3
        rowimg[2 * u * kStep] = (uint8_t)__builtin_amdgcn_udot4(c[u], W, Z, false);
        rowimg[(2 * u + 1) * kStep] = (uint8_t)__builtin_amdgcn_udot4(c[u] >> 16, W, Z, false);
      }
    } else if (L == 3) {
      constexpr uint32_t W = 0x1B090301u;              // bytes {1, 3, 9, 27}
      constexpr uint32_t Z = 0u - (uint32_t)kD * 121u; // the +D of five codes (81 D below)
      const uint32_t* c = reinterpret_cast<const uint32_t*>(crow8);
#pragma unroll
      for (int u = q; u < 26; u += 4) {                // field u = codes 5u .. 5u+4
        const int o = 5 * u;
        const uint32_t d0 = c[o >> 2], d1 = c[(o >> 2) + 1], d2 = c[(o >> 2) + 2];
        const uint32_t x = __builtin_amdgcn_alignbyte(d1, d0, o & 3);
        const uint32_t y = __builtin_amdgcn_alignbyte(d2, d1, o & 3) & 0xFFu;
        rowimg[u * kStep] = (uint8_t)__builtin_amdgcn_udot4(x, W, Z + 81u * y, false);
      }
    } else if (L == 8) {
      constexpr uint32_t W = 0x00400801u;              // bytes {1, 8, 64, 0}
      const uint32_t* c = reinterpret_cast<const uint32_t*>(crow8);
#pragma unroll
      for (int u = q; u < 16; u += 4) {                // codes 8u .. 8u+7 -> bytes 3u .. 3u+2
        const uint32_t x0 = c[2 * u] - kZeroCode, x1 = c[2 * u + 1] - kZeroCode;   // bytes >= D: no borrow
        const uint32_t v = __builtin_amdgcn_udot4(x0, W, 0u, false) | ((x0 >> 24) << 9) |
                           (__builtin_amdgcn_udot4(x1, W, 0u, false) << 12) | ((x1 >> 24) << 21);
        rowimg[3 * u * kStep] = (uint8_t)v;
        rowimg[(3 * u + 1) * kStep] = (uint8_t)(v >> 8);
        rowimg[(3 * u + 2) * kStep] = (uint8_t)(v >> 16);
      }
    } else {
      constexpr uint32_t W = 0x00190501u;              // bytes {1, 5, 25, 0}
      constexpr uint32_t Z = 0u - (uint32_t)kD * 31u;  // removes the +D of three codes
#pragma unroll
      for (int u = q; u < 6; u += 4) {                 // fields 8u .. 8u+7 = bytes 7u .. 7u+6
        const uint32_t* c = reinterpret_cast<const uint32_t*>(crow8 + 24 * u);
        const uint32_t a0 = c[0], a1 = c[1], a2 = c[2], a3 = c[3], a4 = c[4], a5 = c[5];
        uint32_t f[8];
        f[0] = __builtin_amdgcn_udot4(a0, W, Z, false);
        f[1] = __builtin_amdgcn_udot4(__builtin_amdgcn_alignbyte(a1, a0, 3), W, Z, false);
        f[2] = __builtin_amdgcn_udot4(__builtin_amdgcn_alignbyte(a2, a1, 2), W, Z, false);
        f[3] = __builtin_amdgcn_udot4(a2 >> 8, W, Z, false);
        f[4] = __builtin_amdgcn_udot4(a3, W, Z, false);
        f[5] = __builtin_amdgcn_udot4(__builtin_amdgcn_alignbyte(a4, a3, 3), W, Z, false);
        f[6] = __builtin_amdgcn_udot4(__builtin_amdgcn_alignbyte(a5, a4, 2), W, Z, false);
        f[7] = __builtin_amdgcn_udot4(a5 >> 8, W, Z, false);
        if (u == 5) f[3] = f[4] = f[5] = f[6] = f[7] = 0u;   // fields 43.. do not exist
        const uint32_t lo32 = f[0] | (f[1] << 7) | (f[2] << 14) | (f[3] << 21) | (f[4] << 28);
        const uint32_t hi24 = (f[4] >> 4) | (f[5] << 3) | (f[6] << 10) | (f[7] << 17);
        const int nb = u == 5 ? 3 : 7;
        uint8_t* o = rowimg + 7 * u * kStep;
#pragma unroll
        for (int e = 0; e < 7; ++e)
          if (e < nb) o[e * kStep] = (uint8_t)(e < 4 ? lo32 >> (8 * e) : hi24 >> (8 * (e - 4)));
      }
    }
  };
  if (kvsel == 0) pack(std::false_type{});
  else pack(std::true_type{});
  __syncthreads();

  // ---- store the image: slots [slot0, slot0 + nrows) start at byte slot0 * R
  // in both layouts; whole 16-byte pieces (rows past nrows carry zero codes,
  // stay inside the plane and belong to no valid row yet)
  const int bytes = kvsel == 0 ? (nrows * R + 15) & ~15 : ((nrows + 15) >> 4) * 16 * R;
  uint4* dst = reinterpret_cast<uint4*>(a.codes[pool] + plane * a.cap[pool] * R + slot0 * R);
  for (int i = tid; i < (bytes >> 4); i += kThreads)
    store_stream(dst + i, reinterpret_cast<const uint4*>(img)[i]);
}

// One pool's tile: the fast path of its level count (a compile-time count
// when the kernel is specialised for it, else a runtime switch), or the
// generic tile.
template <int LF, bool kRot, bool kRagged>
__device__ __forceinline__ void pool_tile(const QuantArgs& a, int pool, int t, uint8_t* smem) {
  const PoolPart pp = pool_part<kRagged>(a, pool, blockIdx.z);
  if (t * kRows >= pp.count) return;            // past this sequence's rows (ragged bounds)
  const bool aligned16 = (pp.start & 15) == 0;
  const int L = LF ? LF : a.fmt[pool].L;
  uint8_t* img = smem + kCode8Bytes;
  if (aligned16 && fast_quant_level(L)) {
    if (LF == 6 || (LF == 0 && L == 6)) quantize_tile_fast<6, kRot>(a, pp, pool, t, smem, img);
    else if (LF == 5 || (LF == 0 && L == 5)) quantize_tile_fast<5, kRot>(a, pp, pool, t, smem, img);
    else if (LF == 0 && L == 4) quantize_tile_fast<4, kRot>(a, pp, pool, t, smem, img);
    else if (LF == 0 && L == 16) quantize_tile_fast<16, kRot>(a, pp, pool, t, smem, img);
    else if (LF == 0 && L == 8) quantize_tile_fast<8, kRot>(a, pp, pool, t, smem, img);
    else if (LF == 0 && L == 3) quantize_tile_fast<3, kRot>(a, pp, pool, t, smem, img);
  } else {
    quantize_tile<LF, kRot>(a, pp, pool, t, reinterpret_cast<uint16_t*>(smem));
  }
}

template <int LH, int LL, bool kRot, bool kRagged>
__global__ __launch_bounds__(kThreads) void quantize_pack_kernel(QuantArgs a, int tiles_high) {
  constexpr int kGeneric = kRows * kCodeStride * 2;
  constexpr int kFast = kCode8Bytes + kImgBytes;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kGeneric > kFast ? kGeneric : kFast];
  const int tile = blockIdx.x;
  if (tile < tiles_high) pool_tile<LH, kRot, kRagged>(a, 0, tile, smem);
  else pool_tile<LL, kRot, kRagged>(a, 1, tile - tiles_high, smem);
}

// The (6, 5) pair has its own instance; every other pair picks its tiles at
// run time.
template <bool kRagged>
void launch_kind(const QuantArgs& a, dim3 grid, int tiles_high, hipStream_t stream) {
  const bool pair65 = a.fmt[0].L == 6 && a.fmt[1].L == 5;
  if (pair65 && a.rotate)
    hipLaunchKernelGGL((quantize_pack_kernel<6, 5, true, kRagged>), grid, dim3(kThreads), 0, stream, a,
                       tiles_high);
  else if (pair65)
    hipLaunchKernelGGL((quantize_pack_kernel<6, 5, false, kRagged>), grid, dim3(kThreads), 0, stream,
                       a, tiles_high);
  else if (a.rotate)
    hipLaunchKernelGGL((quantize_pack_kernel<0, 0, true, kRagged>), grid, dim3(kThreads), 0, stream, a,
                       tiles_high);
  else
    hipLaunchKernelGGL((quantize_pack_kernel<0, 0, false, kRagged>), grid, dim3(kThreads), 0, stream,
                       a, tiles_high);
}

}  // namespace

hipError_t launch_quantize_pack(const QuantArgs& a, hipStream_t stream) {
  const int count_low = a.n - a.k_high;
  const int tiles_high = (a.k_high + kRows - 1) / kRows;
  const int tiles_low = (count_low + kRows - 1) / kRows;
  const int tiles = tiles_high + tiles_low;
  if (tiles == 0) return hipSuccess;
  dim3 grid(tiles, a.layers * a.kv_heads * 2, a.batch);
  if (a.seq) launch_kind<true>(a, grid, tiles_high, stream);
  else launch_kind<false>(a, grid, tiles_high, stream);
  return hipGetLastError();
}

}  // namespace semkv
