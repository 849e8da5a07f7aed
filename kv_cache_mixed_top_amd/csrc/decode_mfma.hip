// Matrix-core decode attention over pools of 6-level and 5-level rows (the
// SemKV page's operating pair b_high/b_low = log2 6 / log2 5, Fig. 1 and
// Table 2).  Same split-K contract as the generic kernel in decode.hip: one
// workgroup per chunk of one pool plane pair (K and V of one sequence, layer
// and KV head) for the 4 query heads of the KV head, writing (m, l, o[128])
// partials per head.
//
// decode_mfma2_kernel: two waves per chunk.  Wave 0 streams K and computes
// the logits, wave 1 streams V, keeps the softmax and the PV accumulators;
// the logits of a tile pass through LDS with one barrier per tile.
//
// Per 64-row tile:
//  * Staging: direct global->LDS loads of the next tile through a buffer
//    resource over the plane (range-checked, no per-lane address math).
//  * Digits: a field value x enters as the fp16 value 1536 + x (one v_perm
//    puts the byte under a 0x66 high byte); one packed fp16 FMA with the
//    constants below gives 1536 + floor(x / L) exactly, and the digits
//    follow with exact fp16 subtracts and FMAs.  All MFMA operands are
//    normal fp16 values (a chain with subnormal operands measured ~100x
//    larger rounding on gfx950).
//  * QK^T on the 4x4x4 (16-block) f16 MFMA.  Lane t owns token row t of the
//    row-major K plane.  The 4 query heads are the A operand; cbsz = 4
//    broadcasts block `abid`'s A to all 16 blocks, so the q fragments of 16
//    consecutive instructions share one VGPR pair.
//  * logit z = sm_scale * log2(e) * (scale_K * (q . c) + min_K * sum(q)), in
//    log2 units; the weights are taken against a per-head frame a margin
//    above the running maximum, which rises (and rescales the accumulators)
//    only when a logit exceeds it.
//  * PV on the 16x16x32 f16 MFMA with K = 32 tokens.  V planes are stored
//    byte-planar in 16-row tiles (byte j of 16 consecutive rows is
//    contiguous), so one 8-byte LDS read gives one code byte of 8 tokens.
//    The A operand is w = p * scale_V * 2^E (E per chunk keeps w below 2^14)
//    split into two fp16 terms w_hi (A rows 0-3) + w_lo (rows 4-7), so the
//    weights keep ~22 bits: with heavy-tailed V the min_V and scale_V * code
//    terms nearly cancel and a single fp16 weight (11 bits) is not enough.
//    The B operand holds the linear features of each packed field f: f,
//    floor(f/L), floor(f/L^2), centred on integer midpoints of their ranges.
//    The digits are linear in them (c0 = f - L*f1, c1 = f1 - L*f2, c2 = f2),
//    so the digit sums are recovered from the fp32 accumulators at the end;
//    the centring (needed because the weights are all positive: uncentred
//    sums grow with the chunk and the recovery amplifies their rounding)
//    adds coef_k * sum(w) to each digit sum, read from a B column that holds
//    no field.  sum_t p_t * min_V(t) is accumulated on the VALU.
#include <atomic>
#include <utility>

#include "semkv_internal.h"

namespace semkv {
namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 64;
constexpr int kBuf = 3072;          // 3 x 1 KB load blocks (>= 64 * 43 + 48 read slack)
constexpr int kPartialStride = 2 + kHeadDim;
constexpr int kQkInstr = 33;        // 4x4x4 MFMAs per row (132 digit slots)
constexpr float kFrameMargin = 8.0f; // softmax frame above the running max (natural log)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ uint32_t u32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ u16x2 v2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }
__device__ __forceinline__ uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel) {
  return __builtin_amdgcn_perm(s0, s1, sel);
}
__device__ __forceinline__ h4 as_h4(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(h4, make_uint2(lo, hi));
}
__device__ __forceinline__ h8 as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(h8, make_uint4(a, b, c, d));
}

// Field values enter as fp16 in [1024, 2048), where the spacing is 1: a
// 16-bit slot 0x6600 | x is the value 1536 + x (x < 512).  One packed fp16
// FMA then gives 1536 + floor(x / L) exactly: RNE((1536 + x) * m + k) with
// the constants below, checked exhaustively for every field value (x < 216
// for 6 levels, x < 125 for 5) and so also for floor(f1 / L).
constexpr uint32_t kBias = 0x66666666u;   // perm source of the 0x66 high bytes
constexpr float kBase = 1536.0f;
template <int L> constexpr float floor_m() { return L == 6 ? 0.1663818359375f : 0.1995849609375f; }
template <int L> constexpr float floor_k() { return L == 6 ? 1280.0f : 1229.0f; }

template <int L>
__device__ __forceinline__ h2 floor_div(h2 v) {   // 1536 + x -> 1536 + floor(x / L)
  constexpr _Float16 m = (_Float16)floor_m<L>(), k = (_Float16)floor_k<L>();
  return __builtin_elementwise_fma(v, (h2){m, m}, (h2){k, k});
}

// Two biased field values -> their three base-L digits as exact fp16 integers.
template <int L>
__device__ __forceinline__ void digits(uint32_t x, uint32_t& c0, uint32_t& c1, uint32_t& c2) {
  constexpr _Float16 B = (_Float16)kBase, nL = (_Float16)(-L);
  const h2 X = __builtin_bit_cast(h2, x);
  const h2 F1 = floor_div<L>(X);
  const h2 F2 = floor_div<L>(F1);
  const h2 d2 = F2 - (h2){B, B};
  const h2 f1 = F1 - (h2){B, B};
  const h2 d1 = __builtin_elementwise_fma(d2, (h2){nL, nL}, f1);
  const h2 d0 = __builtin_elementwise_fma(f1, (h2){nL, nL}, X - (h2){B, B});
  c0 = __builtin_bit_cast(uint32_t, d0);
  c1 = __builtin_bit_cast(uint32_t, d1);
  c2 = __builtin_bit_cast(uint32_t, d2);
}

// Integer centres of the PV features f, floor(f/L), floor(f/L^2) near the
// middle of their ranges.  The digit sums are then the centred combinations
// plus coef_k * sum(w), coef = (a0 - L a1, a1 - L a2, a2).
template <int L, int K>
constexpr int feature_centre() {
  return L == 6 ? (K == 0 ? 108 : K == 1 ? 18 : 3) : (K == 0 ? 62 : K == 1 ? 12 : 2);
}
template <int L, int K>
constexpr float centre_coef() {
  return K == 0 ? (float)(feature_centre<L, 0>() - L * feature_centre<L, 1>())
       : K == 1 ? (float)(feature_centre<L, 1>() - L * feature_centre<L, 2>())
                : (float)feature_centre<L, 2>();
}

// Two biased field values -> their centred features as exact fp16 integers.
template <int L>
__device__ __forceinline__ void features(uint32_t x, uint32_t& g0, uint32_t& g1, uint32_t& g2) {
  constexpr _Float16 a0 = (_Float16)(kBase + feature_centre<L, 0>());
  constexpr _Float16 a1 = (_Float16)(kBase + feature_centre<L, 1>());
  constexpr _Float16 a2 = (_Float16)(kBase + feature_centre<L, 2>());
  const h2 X = __builtin_bit_cast(h2, x);
  const h2 F1 = floor_div<L>(X);
  const h2 F2 = floor_div<L>(F1);
  g0 = __builtin_bit_cast(uint32_t, X - (h2){a0, a0});
  g1 = __builtin_bit_cast(uint32_t, F1 - (h2){a1, a1});
  g2 = __builtin_bit_cast(uint32_t, F2 - (h2){a2, a2});
}

// Query fragments of the QK^T product (ABID-packed 4x4x4 A operands).  With
// kLo (a rotated cache) the query is the fp32 rotation H q, carried as its
// nearest fp16 `hi` plus the fp16 remainder `lo` (about 22 bits), so that the
// logits do not inherit an fp16 rounding of H q; each product then takes one
// more MFMA into the same accumulator.
template <bool kLo>
struct QFrag {
  h4 hi[3];
  h4 lo[kLo ? 3 : 1];
};

template <int S, bool kLo>
__device__ __forceinline__ f4 qk_mfma(const QFrag<kLo>& qf, uint32_t lo, uint32_t hi, f4 acc) {
  acc = __builtin_amdgcn_mfma_f32_4x4x4f16(qf.hi[S / 16], as_h4(lo, hi), acc, 4, S % 16, 0);
  if constexpr (kLo)
    acc = __builtin_amdgcn_mfma_f32_4x4x4f16(qf.lo[S / 16], as_h4(lo, hi), acc, 4, S % 16, 0);
  return acc;
}

// ---- 6 levels: one K row = 43 bytes = 11 dwords (the 44th byte masked)
template <int W, int NC, bool kLo>
__device__ __forceinline__ void qk6_dword(const uint32_t (&d)[12], const QFrag<kLo>& qf,
                                          f4 (&acc)[3]) {
  const uint32_t X = d[W];
  const uint32_t xe = perm(kBias, X, 0x04020400u);   // bytes 4W, 4W+2 -> biased slots
  const uint32_t xo = perm(kBias, X, 0x04030401u);   // bytes 4W+1, 4W+3
  uint32_t e0, e1, e2, o0, o1, o2;
  digits<6>(xe, e0, e1, e2);
  digits<6>(xo, o0, o1, o2);
  acc[0 % NC] = qk_mfma<3 * W + 0, kLo>(qf, e0, o0, acc[0 % NC]);
  acc[1 % NC] = qk_mfma<3 * W + 1, kLo>(qf, e1, o1, acc[1 % NC]);
  acc[2 % NC] = qk_mfma<3 * W + 2, kLo>(qf, e2, o2, acc[2 % NC]);
}
template <int NC, bool kLo, int... Ws>
__device__ __forceinline__ void qk6(const uint32_t (&d)[12], const QFrag<kLo>& qf, f4 (&acc)[3],
                                    std::integer_sequence<int, Ws...>) {
  (qk6_dword<Ws, NC, kLo>(d, qf, acc), ...);
}

// ---- 5 levels: one K row = 38 bytes; 7-byte units hold 8 fields of 7 bits.
// From a word W with fields at bits 0, 7, 14, 21: slots (F0, F2) and (F1, F3).
// `bias` is 0x66006600 held in a register, so that each mask and OR is one
// AND-OR.  The 16-bit halves (W[0:15], W[14:29]) hold F0 and F2 in their low
// 7 bits, and F1 and F3 seven bits higher.
__device__ __forceinline__ void field_pairs(uint32_t W, uint32_t& pa, uint32_t& pb,
                                            uint32_t bias) {
  const uint32_t h = perm(W >> 14, W, 0x05040100u);
  pa = (h & 0x007F007Fu) | bias;                                       // (F0, F2)
  const u16x2 seven = {7, 7};
  pb = (u32(v2(h) >> seven) & 0x007F007Fu) | bias;                     // (F1, F3)
}
// 0x66006600 in a vector register (the compiler cannot fold it back into a
// literal, which these instructions cannot take together with a mask).
__device__ __forceinline__ uint32_t bias_register() {
  uint32_t b;
  asm volatile("v_mov_b32 %0, 0x66006600" : "=v"(b));
  return b;
}
template <int Q, int NC, bool kLo>   // Q = 2u + quad
__device__ __forceinline__ void qk5_quad(uint32_t W, const QFrag<kLo>& qf, f4 (&acc)[3],
                                         uint32_t bias) {
  uint32_t pa, pb, a0, a1, a2, b0, b1, b2;
  field_pairs(W, pa, pb, bias);
  digits<5>(pa, a0, a1, a2);
  digits<5>(pb, b0, b1, b2);
  acc[0 % NC] = qk_mfma<3 * Q + 0, kLo>(qf, a0, b0, acc[0 % NC]);
  acc[1 % NC] = qk_mfma<3 * Q + 1, kLo>(qf, a1, b1, acc[1 % NC]);
  acc[2 % NC] = qk_mfma<3 * Q + 2, kLo>(qf, a2, b2, acc[2 % NC]);
}
template <int U, int NC, bool kLo>
__device__ __forceinline__ void qk5_unit(const uint32_t (&d)[12], const QFrag<kLo>& qf,
                                         f4 (&acc)[3], uint32_t bias) {
  constexpr int b0 = 7 * U;
  const uint32_t lo = __builtin_amdgcn_alignbyte(d[b0 / 4 + 1], d[b0 / 4], b0 % 4);
  if (U < 5) {
    constexpr int b1 = 7 * U + 4;
    const uint32_t hi = __builtin_amdgcn_alignbyte(d[b1 / 4 + 1], d[b1 / 4], b1 % 4);
    const uint32_t m = __builtin_amdgcn_alignbit(hi, lo, 28);
    qk5_quad<2 * U, NC, kLo>(lo, qf, acc, bias);
    qk5_quad<2 * U + 1, NC, kLo>(m, qf, acc, bias);
  } else {
    qk5_quad<2 * U, NC, kLo>(lo, qf, acc, bias);   // fields 40..42 and one zero pad field
  }
}
template <int NC, bool kLo, int... Us>
__device__ __forceinline__ void qk5(const uint32_t (&d)[12], const QFrag<kLo>& qf, f4 (&acc)[3],
                                    uint32_t bias, std::integer_sequence<int, Us...>) {
  (qk5_unit<Us, NC, kLo>(d, qf, acc, bias), ...);
}

// d index of slot `i` (0..3) of QK instruction s, or -1 for a zero slot.
template <int L>
__device__ __forceinline__ int qk_slot_dim(int s, int i) {
  const int order[4] = {0, 2, 1, 3};
  if (L == 6) {
    const int w = s / 3, k = s % 3;
    const int byte = 4 * w + order[i];
    const int d = 3 * byte + k;
    return (byte < 43 && d < kHeadDim) ? d : -1;
  } else {
    const int q = s / 3, k = s % 3;           // q = 2u + quad
    const int f = 4 * q + order[i];           // fields 8u + 4quad + {0,2,1,3}
    const int d = 3 * f + k;
    return (f < 43 && d < kHeadDim) ? d : -1;
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

// Largest V scale (the low half of the meta word) over rows [r0, r1), as
// fp16 bits, in every lane.  r0 is a multiple of 4 and the meta plane is
// 16-byte aligned, so the rows are read four to a 16-byte load, sixteen loads
// per lane in flight: a chunk of up to 4096 rows costs one memory latency.
__device__ __forceinline__ uint32_t chunk_scale_max(const uint32_t* vmg, int64_t r0, int64_t r1,
                                                    int lane) {
  constexpr int kDepth = 16;
  uint32_t smax = 0;
  const int64_t n4 = (r1 - r0) >> 2;
  const uint4* g4 = reinterpret_cast<const uint4*>(vmg + r0);
  for (int64_t i = lane; i < n4; i += 64 * kDepth) {
    uint4 v[kDepth];
#pragma unroll
    for (int k = 0; k < kDepth; ++k) v[k] = g4[min(i + 64 * k, n4 - 1)];   // repeats are harmless
#pragma unroll
    for (int k = 0; k < kDepth; ++k)
      smax = max(smax, max(max(v[k].x & 0xFFFFu, v[k].y & 0xFFFFu), max(v[k].z & 0xFFFFu, v[k].w & 0xFFFFu)));
  }
  const int64_t rr = r0 + 4 * n4 + lane;           // the last (r1 - r0) % 4 rows
  if (rr < r1) smax = max(smax, vmg[rr] & 0xFFFFu);
  return wave_max_u32(smax);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
// LDS address of byte `off` of a shared buffer; the offset is added in the
// LDS address space, so the DMA target stays visibly inside its buffer.
__device__ __forceinline__ lds_void* lds_at(uint8_t* p, int off) { return (lds_void*)((lds_u8*)p + off); }

// Partial record of a chunk: per-head sums, digit sums from the feature
// sums, (m, l, o[128]) per query head.
template <int L>
__device__ __forceinline__ void write_partial(const DecodeArgs& a, int64_t u, int lane, int E,
                                              f4 (&acc)[3][3], const float (&mref)[4],
                                              float (&lsum)[4], float (&msum)[4],
                                              float m_unit = 1.0f) {
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    lsum[h] = wave_sum(lsum[h]);
    msum[h] = wave_sum(msum[h]);
  }
  // C rows 4-7 (lanes 16-31) hold the w_lo products of the heads in rows 0-3
#pragma unroll
  for (int set = 0; set < 3; ++set)
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[set][k][r] += __shfl_xor(acc[set][k][r], 16, 64);
  // Centred features: every digit sum is its centred combination plus
  // coef_k * sum(w).  Column 15 of set 2 (field 47) holds no field: its
  // features are 0, centred -a_k, so its feature-2 sum is -a2 * sum(w).
  float wsum[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    wsum[r] = __shfl(acc[2][2][r], 15, 64) * (-1.0f / (float)feature_centre<L, 2>());
  float* wsu = a.ws + u * 4 * kPartialStride;
  const float back = ldexpf(1.0f, -E);       // undo the chunk exponent of w
  if (lane < 16) {
#pragma unroll
    for (int set = 0; set < 3; ++set) {
      const int j = 16 * set + lane;
      if (j < 43) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float F0 = acc[set][0][r] * back;
          const float F1 = acc[set][1][r] * back;
          const float F2 = acc[set][2][r] * back;
          const float W = wsum[r] * back;
          float* o = wsu + r * kPartialStride + 2;
          const int d = 3 * j;
          o[d] = msum[r] + fmaf(centre_coef<L, 0>(), W, fmaf(-(float)L, F1, F0));
          o[d + 1] = msum[r] + fmaf(centre_coef<L, 1>(), W, fmaf(-(float)L, F2, F1));
          if (d + 2 < kHeadDim) o[d + 2] = msum[r] + fmaf(centre_coef<L, 2>(), W, F2);
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < 4; ++h)
    if (lane == h) {
      wsu[h * kPartialStride + 0] = mref[h] * m_unit;   // natural-log units
      wsu[h * kPartialStride + 1] = lsum[h];
    }
}

// ---- two-wave form: one workgroup of two waves per chunk.  Wave 0 streams
// the K rows and computes the logits; wave 1 streams the V tiles, keeps the
// softmax and the PV accumulators and writes the partial record.  The
// logits of a tile pass through LDS (double-buffered) with one workgroup
// barrier per tile, so wave 0 computes tile t+1 while wave 1 finishes tile
// t, and each wave holds only its own half of the state.
// The buffers are separate LDS arrays (pointers into them are selected by
// tile parity), so that an LDS access can be told apart from an in-flight
// global->LDS load into another buffer; otherwise the compiler waits for the
// loads before it.
struct Stage2 {
  uint8_t *k0, *k1;            // wave 0 staging, kBuf bytes each
  uint8_t *v0, *v1;            // wave 1 staging
  float *z0, *z1;              // logits of the last two tiles, [4][kTile] + maxima [4]
  _Float16* w;                 // wave 1: weights hi, lo, [2 * 4 * kTile]
  _Float16* qr;                // wave 0: the rotated queries of a rotated cache, hi and
                               // lo, [2][4][128]
  __device__ uint8_t* k(int b) const { return b ? k1 : k0; }
  __device__ uint8_t* v(int b) const { return b ? v1 : v0; }
  __device__ float* z(int b) const { return b ? z1 : z0; }
};

// One workgroup barrier with no memory fence: the LDS writes before it are
// waited for by the caller; outstanding global->LDS prefetches stay in flight.
__device__ __forceinline__ void tile_barrier() { asm volatile("s_barrier" ::: "memory"); }
// 16-byte LDS read that also waits for it (and every LDS access before it)
// inside the same asm block, so that the result register is written when
// the block ends.  Used where the compiler cannot tell the read apart from
// global->LDS loads in flight into other buffers and would wait for those.
__device__ __forceinline__ h8 lds_read_h8_wait(const _Float16* p) {
  h8 r;
  const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) _Float16*)p;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(a) : "memory");
  return r;
}
// s_waitcnt through the builtin (not inline asm), so that the compiler's own
// wait insertion knows what has completed; the encodings are those of the
// CDNA s_waitcnt immediate (vmcnt in bits 3:0 and 15:14, expcnt in 6:4,
// lgkmcnt in 11:8).
// Raw buffer resource over `bytes` bytes from `base` (CDNA buffer
// descriptor, stride 0): loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t plane_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

template <int L, bool kRot>
__device__ __forceinline__ void qk_wave(const DecodeArgs& a, int seg, int64_t r0, int64_t r1, int b, int li,
                        int g, Stage2& st) {
  constexpr int R = (L == 6) ? 43 : 38;
  const int lane = threadIdx.x & 63;
  const int layer = a.layer0 + li;
  const int64_t plane_k = (((int64_t)b * a.layers + layer) * a.kv_heads + g) * 2;
  const int cap = (int)a.cap[seg];            // cap * R < 2^31 (checked by the launcher)
  const int ir0 = (int)r0, ir1 = (int)r1;
  const uint8_t* kcodes = a.codes[seg] + plane_k * cap * R;
  const uint32_t* kmg = a.meta[seg] + plane_k * cap;
  const float sm = a.sm_scale * kLog2e;   // logits in log2 units
  const uint32_t bias5 = L == 5 ? bias_register() : 0u;   // 5-level field bias

  // queries: ABID-packed 4x4x4 A fragments and per-head sums (loaded once
  // the first K tile is in flight)
  QFrag<kRot> qf;
  float sumq[4];
  // The 3 KB of K bytes from row t0 on -> buffer `buf` (16 bytes per lane per
  // instruction), and the lane's K meta word -> register.  The plane from
  // row t0 is a buffer resource built on the scalar unit: the loads need no
  // per-lane address arithmetic, and bytes past the plane read as zeros (the
  // rows past the tile are not used).
  uint32_t km_next = 0;
  const uint32_t lane16 = 16u * (uint32_t)lane;
  auto issue = [&](int buf, int t0) {
    const __amdgpu_buffer_rsrc_t rk = plane_rsrc(kcodes + t0 * R, (cap - t0) * R);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, lds_at(st.k(buf), 0), 16, (int)lane16, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, lds_at(st.k(buf), 0), 16, (int)lane16, 0, 1024, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, lds_at(st.k(buf), 0), 16, (int)lane16, 0, 2048, 0);
    km_next = __builtin_amdgcn_raw_buffer_load_b32(plane_rsrc(kmg + t0, (cap - t0) * 4), 4 * lane, 0, 0);
  };

  float frame[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  // One tile in staging buffer B (a compile-time constant, so that reads of
  // buffer B are known not to overlap the loads in flight into 1 - B).
  auto tile = [&](int t0, auto Bc) {
    constexpr int B = decltype(Bc)::value;
    const int nt = min(kTile, ir1 - t0);
    wait_vm0();   // this tile's rows have landed
    const uint32_t km = km_next;
    if (t0 + kTile < ir1) issue(1 - B, t0 + kTile);
    f4 sacc[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) sacc[k] = (f4){0.f, 0.f, 0.f, 0.f};
    {
      const int off = lane * R;
      const uint32_t* kb32 = reinterpret_cast<const uint32_t*>(st.k(B) + (off & ~3));
      const int sh = off & 3;
      uint32_t d[12];
#pragma unroll
      for (int i = 0; i < 11; ++i) d[i] = __builtin_amdgcn_alignbyte(kb32[i + 1], kb32[i], sh);
      d[11] = 0;
      if (L == 6) {
        d[10] &= 0x00FFFFFFu;                       // byte 43 belongs to the next row
        qk6<1, kRot>(d, qf, sacc, std::make_integer_sequence<int, 11>{});
      } else {
        d[9] &= 0x0000FFFFu;                        // bytes 38, 39 belong to the next row
        d[10] = 0;
        qk5<1, kRot>(d, qf, sacc, bias5, std::make_integer_sequence<int, 6>{});
      }
    }
    const float kfac = sm * h2f((uint16_t)(km & 0xFFFFu));
    const float kbias = sm * h2f((uint16_t)(km >> 16));
    float z[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) z[h] = fmaf(kfac, sacc[0][h], kbias * sumq[h]);   // one accumulator chain
    if (nt < kTile) {                          // rows past the chunk end take no weight
#pragma unroll
      for (int h = 0; h < 4; ++h) z[h] = lane < nt ? z[h] : -INFINITY;
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) st.z(B)[h * kTile + lane] = z[h];
    // softmax frame per head, kFrameMargin above the running maximum; it is
    // raised only when a logit exceeds it (in practice on the first tile)
    const bool up = z[0] > frame[0] || z[1] > frame[1] || z[2] > frame[2] || z[3] > frame[3];
    if (__ballot(up) != 0ull) {
#pragma unroll
      for (int h = 0; h < 4; ++h) frame[h] = fmaxf(frame[h], wave_max(z[h]) + kFrameMargin * kLog2e);
    }
    if (lane == 0)
      *reinterpret_cast<float4*>(st.z(B) + 4 * kTile) =
          make_float4(frame[0], frame[1], frame[2], frame[3]);
    wait_lgkm0();  // logits written
    tile_barrier();
  };
  if (ir0 < ir1) issue(0, ir0);
  const _Float16* qg = reinterpret_cast<const _Float16*>(a.q) +
                       (((int64_t)b * a.nl + li) * a.q_heads + g * 4) * kHeadDim;
  // A fragments of the 4 heads' query values at `qs`
  auto fragments = [&](const _Float16* qs, h4 (&out)[3]) {
    const int head = lane & 3, blk = lane >> 2;
#pragma unroll
    for (int P = 0; P < 3; ++P) {
      const int s = 16 * P + blk;
      h4 v = {0, 0, 0, 0};
      if (s < kQkInstr) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = qk_slot_dim<L>(s, i);
          v[i] = d >= 0 ? qs[head * kHeadDim + d] : (_Float16)0.0f;
        }
      }
      out[P] = v;
    }
  };
  if constexpr (kRot) {
    // rotated cache: q -> H q in fp32 (lane holds dimensions 2 lane, 2 lane + 1:
    // index bit 0 within the lane, bits 1-6 across lanes), carried as the
    // nearest fp16 plus the fp16 remainder; sum(H q) for the min term is
    // taken from the fp32 values
    constexpr float kNorm = 0.08838834764831845f;   // 1/sqrt(128)
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float x0 = (float)qg[h * kHeadDim + 2 * lane], x1 = (float)qg[h * kHeadDim + 2 * lane + 1];
      float y0 = x0 + x1, y1 = x0 - x1;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const float p0 = __shfl_xor(y0, m, 64), p1 = __shfl_xor(y1, m, 64);
        const bool upper = (lane & m) != 0;
        y0 = upper ? p0 - y0 : y0 + p0;
        y1 = upper ? p1 - y1 : y1 + p1;
      }
      y0 *= kNorm;
      y1 *= kNorm;
      const _Float16 h0 = (_Float16)y0, h1 = (_Float16)y1;
      st.qr[h * kHeadDim + 2 * lane] = h0;
      st.qr[h * kHeadDim + 2 * lane + 1] = h1;
      st.qr[(4 + h) * kHeadDim + 2 * lane] = (_Float16)(y0 - (float)h0);
      st.qr[(4 + h) * kHeadDim + 2 * lane + 1] = (_Float16)(y1 - (float)h1);
      sumq[h] = wave_sum(y0 + y1);
    }
    wait_lgkm0();   // the wave's LDS writes have landed
    fragments(st.qr, qf.hi);
    fragments(st.qr + 4 * kHeadDim, qf.lo);
  } else {
    fragments(qg, qf.hi);
#pragma unroll
    for (int h = 0; h < 4; ++h)
      sumq[h] = wave_sum((float)qg[h * kHeadDim + 2 * lane] + (float)qg[h * kHeadDim + 2 * lane + 1]);
  }

  for (int t0 = ir0; t0 < ir1; t0 += 2 * kTile) {   // same tile sequence as wave 1
    tile(t0, std::integral_constant<int, 0>{});
    if (t0 + kTile < ir1) tile(t0 + kTile, std::integral_constant<int, 1>{});
  }
}

template <int L>
__device__ __forceinline__ void pv_wave(const DecodeArgs& a, int seg, int64_t r0, int64_t r1, int b, int li,
                        int g, int64_t u, Stage2& st) {
  constexpr int R = (L == 6) ? 43 : 38;
  const int lane = threadIdx.x & 63;
  _Float16* wbuf = st.w;
  const int layer = a.layer0 + li;
  const int64_t plane_k = (((int64_t)b * a.layers + layer) * a.kv_heads + g) * 2;
  const int cap = (int)a.cap[seg];            // cap * R < 2^31 (checked by the launcher)
  const int ir0 = (int)r0, ir1 = (int)r1;
  const uint8_t* vcodes = a.codes[seg] + (plane_k + 1) * cap * R;
  const uint32_t* vmg = a.meta[seg] + (plane_k + 1) * cap;

  // per-chunk exponent E: w = p * scale_V * 2^E stays below 2^14 (set
  // below, once the first V tile is in flight)
  int E = 0;
  float two_e = 1.0f;

  float mref[4], lsum[4], msum[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    mref[h] = -INFINITY;
    lsum[h] = 0.f;
    msum[h] = 0.f;
  }
  f4 acc[3][3];
#pragma unroll
  for (int s = 0; s < 3; ++s)
#pragma unroll
    for (int k = 0; k < 3; ++k) acc[s][k] = (f4){0.f, 0.f, 0.f, 0.f};

  // The 3 KB of V bytes (16-row byte-planar tiles) from row t0 on -> buffer
  // `buf`, and the lane's V meta word -> register, through buffer resources
  // as in the K wave
  uint32_t vm_next = 0;
  const uint32_t lane16 = 16u * (uint32_t)lane;
  auto issue = [&](int buf, int t0) {
    const __amdgpu_buffer_rsrc_t rv = plane_rsrc(vcodes + t0 * R, (cap - t0) * R);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, lds_at(st.v(buf), 0), 16, (int)lane16, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, lds_at(st.v(buf), 0), 16, (int)lane16, 0, 1024, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, lds_at(st.v(buf), 0), 16, (int)lane16, 0, 2048, 0);
    vm_next = __builtin_amdgcn_raw_buffer_load_b32(plane_rsrc(vmg + t0, (cap - t0) * 4), 4 * lane, 0, 0);
  };

  const int col = lane & 15;
  const int quad = lane >> 4;
  // the 0x66 bias bytes of 5-level fields, held in a register so that the
  // mask and the bias go into one AND-OR
  const uint32_t bias5 = L == 5 ? bias_register() : 0u;
  // One tile in staging buffer B (a compile-time constant, so that reads of
  // buffer B are known not to overlap the loads in flight into 1 - B: the
  // next tile's loads go out first and the V bytes are read where used).
  auto tile = [&](int t0, auto Bc) {
    constexpr int B = decltype(Bc)::value;
    const int nt = min(kTile, ir1 - t0);
    wait_vm0();   // this tile's V has landed
    const uint32_t vm = vm_next;
    if (t0 + kTile < ir1) issue(1 - B, t0 + kTile);
    tile_barrier();                                      // logits of this tile are in LDS
    float z[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) z[h] = st.z(B)[h * kTile + lane];
    const float4 fr = *reinterpret_cast<const float4*>(st.z(B) + 4 * kTile);   // all lanes alike

    // the weights are taken against the frame of wave 0; when it was raised
    // (in practice only on the first tile) what was accumulated is rescaled
    if (fr.x != mref[0] || fr.y != mref[1] || fr.z != mref[2] || fr.w != mref[3]) {
      const float nf[4] = {fr.x, fr.y, fr.z, fr.w};
      float fac[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        fac[h] = __builtin_amdgcn_exp2f(mref[h] - nf[h]);   // 2^-inf = 0 on the first tile
        mref[h] = nf[h];
        lsum[h] *= fac[h];
        msum[h] *= fac[h];
      }
#pragma unroll
      for (int s = 0; s < 3; ++s)
#pragma unroll
        for (int k = 0; k < 3; ++k)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[s][k][r] *= fac[r];
    }
    const float vs = h2f((uint16_t)(vm & 0xFFFFu)) * two_e;
    const float vmin = h2f((uint16_t)(vm >> 16));
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float p = __builtin_amdgcn_exp2f(z[h] - mref[h]);
      lsum[h] += p;
      msum[h] = fmaf(p, vmin, msum[h]);
      const float w = p * vs;
      const _Float16 whi = (_Float16)w;
      wbuf[h * kTile + lane] = whi;
      wbuf[4 * kTile + h * kTile + lane] = (_Float16)(w - (float)whi);
    }
    wait_lgkm0();  // weights visible to the wave

    // PV: 32 tokens per MFMA
    const uint8_t* vbuf = st.v(B);
#pragma unroll
    for (int G = 0; G < 2; ++G) {
      if (32 * G >= nt) break;
      // A rows 0-3: w_hi of the 4 heads, rows 4-7: w_lo; rows 8-15 repeat
      // them and only feed C rows 8-15, which are never read.
      const h8 aw = lds_read_h8_wait(wbuf + (col & 7) * kTile + 32 * G + 8 * quad);
      const int tok0 = 32 * G + 8 * quad;
      const int vo = (tok0 >> 4) * (16 * R) + (tok0 & 15);
#pragma unroll
      for (int set = 0; set < 3; ++set) {
        const int j = 16 * set + col;                     // byte (L=6) or field (L=5)
        // this lane's code byte(s) of 8 tokens
        uint32_t p0, p1, p2, p3;
        if (L == 6) {
          const uint2 w8 = j < R ? *reinterpret_cast<const uint2*>(vbuf + (vo + j * 16)) : make_uint2(0u, 0u);
          p0 = perm(kBias, w8.x, 0x04010400u);
          p1 = perm(kBias, w8.x, 0x04030402u);
          p2 = perm(kBias, w8.y, 0x04010400u);
          p3 = perm(kBias, w8.y, 0x04030402u);
        } else {
          const int j0 = (7 * j) >> 3;
          const bool ok = j < 43;
          const uint2 b0 = ok ? *reinterpret_cast<const uint2*>(vbuf + (vo + j0 * 16)) : make_uint2(0u, 0u);
          const uint2 b1 = ok ? *reinterpret_cast<const uint2*>(vbuf + (vo + (j0 + 1) * 16)) : make_uint2(0u, 0u);
          const int bit = 7 * j;
          const u16x2 shv = {(unsigned short)(bit & 7), (unsigned short)(bit & 7)};
          p0 = (u32(v2(perm(b1.x, b0.x, 0x05010400u)) >> shv) & 0x007F007Fu) | bias5;
          p1 = (u32(v2(perm(b1.x, b0.x, 0x07030602u)) >> shv) & 0x007F007Fu) | bias5;
          p2 = (u32(v2(perm(b1.y, b0.y, 0x05010400u)) >> shv) & 0x007F007Fu) | bias5;
          p3 = (u32(v2(perm(b1.y, b0.y, 0x07030602u)) >> shv) & 0x007F007Fu) | bias5;
        }
        uint32_t g0[4], g1[4], g2[4];
        features<L>(p0, g0[0], g1[0], g2[0]);
        features<L>(p1, g0[1], g1[1], g2[1]);
        features<L>(p2, g0[2], g1[2], g2[2]);
        features<L>(p3, g0[3], g1[3], g2[3]);
        const h8 B0 = as_h8(g0[0], g0[1], g0[2], g0[3]);
        const h8 B1 = as_h8(g1[0], g1[1], g1[2], g1[3]);
        const h8 B2 = as_h8(g2[0], g2[1], g2[2], g2[3]);
        acc[set][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, B0, acc[set][0], 0, 0, 0);
        acc[set][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, B1, acc[set][1], 0, 0, 0);
        acc[set][2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, B2, acc[set][2], 0, 0, 0);
      }
    }
  };
  if (ir0 < ir1) issue(0, ir0);
  {
    const uint32_t smax = chunk_scale_max(vmg, r0, r1, lane);
    if (smax != 0) E = 13 - ilogbf(h2f((uint16_t)smax));
    two_e = ldexpf(1.0f, E);
  }
  for (int t0 = ir0; t0 < ir1; t0 += 2 * kTile) {   // same tile sequence as wave 0
    tile(t0, std::integral_constant<int, 0>{});
    if (t0 + kTile < ir1) tile(t0 + kTile, std::integral_constant<int, 1>{});
  }
  write_partial<L>(a, u, lane, E, acc, mref, lsum, msum, kLn2);
}

template <bool kRot>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(4, 8))) void decode_mfma2_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t k0[kBuf], k1[kBuf], v0[kBuf], v1[kBuf];
  __shared__ __attribute__((aligned(16))) float z0[4 * kTile + 4], z1[4 * kTile + 4];
  __shared__ __attribute__((aligned(16))) _Float16 w[2 * 4 * kTile];
  __shared__ __attribute__((aligned(16))) _Float16 qr[kRot ? 2 * 4 * kHeadDim : 8];
  Stage2 st;
  st.qr = qr;
  st.k0 = k0;
  st.k1 = k1;
  st.v0 = v0;
  st.v1 = v1;
  st.z0 = z0;
  st.z1 = z1;
  st.w = w;

  const int x = blockIdx.x;
  const int seg = x < a.nch[0] ? 0 : 1;
  const int ch = seg == 0 ? x : x - a.nch[0];
  const int64_t r0 = (int64_t)ch * a.chunk;
  const int64_t r1 = min(r0 + (int64_t)a.chunk, a.rows[seg]);
  const int li = blockIdx.y / a.kv_heads;
  const int g = blockIdx.y % a.kv_heads;
  const int b = blockIdx.z;
  const int64_t u = (((int64_t)b * a.nl + li) * a.kv_heads + g) * a.nchunks + x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (a.fmt[seg].L == 6) {
    if (wave == 0) qk_wave<6, kRot>(a, seg, r0, r1, b, li, g, st);
    else pv_wave<6>(a, seg, r0, r1, b, li, g, u, st);
  } else {
    if (wave == 0) qk_wave<5, kRot>(a, seg, r0, r1, b, li, g, st);
    else pv_wave<5>(a, seg, r0, r1, b, li, g, u, st);
  }
}

}  // namespace

// Workgroups of the matrix-core kernel resident on the current device at
// once (registers and LDS both limit it); the pool chunking fills them once.
// Cached per device ordinal; concurrent first calls compute the same value.
int64_t decode_mfma_resident_waves() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int64_t> slots[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 2048;
  if (dev < kMaxDevices) {
    const int64_t v = slots[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0, per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_mfma2_kernel<false>, 128, 0) !=
          hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0 || per_cu <= 0)
    return 2048;
  const int64_t v = (int64_t)cus * per_cu;
  if (dev < kMaxDevices) slots[dev].store(v, std::memory_order_relaxed);
  return v;
}

bool decode_mfma_supported(const DecodeArgs& a) {
  if (a.group != 4) return false;
  for (int s = 0; s < 2; ++s) {
    if (a.rows[s] > 0 && a.fmt[s].L != 5 && a.fmt[s].L != 6) return false;
    if (a.cap[s] * 43 >= ((int64_t)1 << 31)) return false;   // 32-bit row offsets in the kernels
  }
  return true;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
  const int pool_chunks = a.nch[0] + a.nch[1];
  if (pool_chunks == 0) return hipSuccess;
  dim3 grid(pool_chunks, a.nl * a.kv_heads, a.batch);
  if (a.rotate)
    hipLaunchKernelGGL(decode_mfma2_kernel<true>, grid, dim3(128), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_mfma2_kernel<false>, grid, dim3(128), 0, stream, a);
  return hipGetLastError();
}

}  // namespace semkv
