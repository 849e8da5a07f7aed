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
//  * Floors: a field value x enters as the fp16 value 1536 + x (one v_perm
//    puts the byte under a 0x66 high byte); one packed fp16 FMA with the
//    constants below gives 1536 + floor(x / L) exactly, applied twice for
//    floor(x / L^2).
//  * QK^T on the int8 matrix cores (16x16x64): the features x, floor(x/L),
//    floor(x/L^2) of every field against a transformed fixed-point query in
//    four signed limbs, products and sums exact in int32 (see qk_wave_i8).
//  * logit z = sm_scale * log2(e) * (scale_K * (q . c) + min_K * sum(q)), in
//    log2 units; the weights are taken against a per-head frame a margin
//    above the running maximum, which rises (and rescales the accumulators)
//    only when a logit exceeds it.
//  * PV on the 16x16x32 f16 MFMA with K = 32 tokens.  V planes are stored
//    byte-planar in 16-row tiles (byte j of 16 consecutive rows is
//    contiguous), so one 8-byte LDS read gives one code byte of 8 tokens.
//    The A operand is w = p * scale_V * 2^E (E per chunk, from the first
//    tile's largest scale and lowered if a later tile needs it, keeps w
//    below 2^15) split into two fp16 terms w_hi (A rows 0-3) + w_lo (rows
//    4-7), so the weights keep ~22 bits: with heavy-tailed V the min_V and
//    scale_V * code terms nearly cancel and a single fp16 weight (11 bits)
//    is not enough.  All f16 MFMA operands are normal fp16 values (a chain
//    with subnormal operands measured ~100x larger rounding on gfx950).
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

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 64;
constexpr int kBuf = 3072;          // 3 x 1 KB load blocks (>= 64 * 43 + 48 read slack)
constexpr int kPartialStride = 2 + kHeadDim;
constexpr float kFrameMargin = 8.0f; // softmax frame above the running max (natural log)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ uint32_t u32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ u16x2 v2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }
__device__ __forceinline__ uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel) {
  return __builtin_amdgcn_perm(s0, s1, sel);
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

// ---- two-wave form: one workgroup of two waves per chunk.  Wave 0 loads
// the tiles and computes the logits; wave 1 keeps the softmax and the PV
// accumulators and writes the partial record.  Per 64-row tile there is one
// workgroup barrier: before it wave 0 has written the tile's logits to LDS
// and its V bytes have landed in LDS; after it wave 1 consumes both while
// wave 0 goes on with the next tile.
//
// Staging, two tiles ahead, all issued by wave 0 in this order per tile:
// the V bytes go global->LDS into one of three buffers (read only by wave
// 1), then the K rows and K meta go straight into registers (three register
// slots).  Loads complete in issue order, so once wave 0 has its K rows of
// tile t (the compiler waits for those registers before it uses them), the
// V bytes of tile t are in LDS too; the barrier after the logits hands them
// to wave 1.  The V buffer of tile t + 2 is the one wave 1 finished before
// it reached the barrier of tile t, so wave 0 refills it after that barrier.
// Wave 1 issues only its V meta loads (registers, two tiles ahead) and so
// needs no wait for global->LDS loads before its LDS reads.  Tile slots are
// compile-time constants (the loop is unrolled by three), and the loads of a
// tile past the chunk go through an empty buffer range: they read nothing,
// and every tile issues the same instructions.
struct Stage3 {
  uint8_t *v0, *v1, *v2;       // V tiles, kBuf bytes each
  float *z0, *z1, *z2;         // logits [4][kTile] + frames [4]
  _Float16* w;                 // wave 1: weights hi, lo, [2 * 4 * kTile]
};
template <int S> __device__ __forceinline__ uint8_t* vbuf_of(const Stage3& st) {
  return S == 0 ? st.v0 : S == 1 ? st.v1 : st.v2;
}
template <int S> __device__ __forceinline__ float* zbuf_of(const Stage3& st) {
  return S == 0 ? st.z0 : S == 1 ? st.z1 : st.z2;
}
template <int S> using Slot = std::integral_constant<int, S>;

// Tiles 0 .. n-1 in slots 0, 1, 2, 0, ...: step(Slot<S>, tile) for each.
template <typename F>
__device__ __forceinline__ void for_tiles(int n, F&& step) {
  int v = 0;
  for (; v + 3 <= n; v += 3) {
    step(Slot<0>{}, v);
    step(Slot<1>{}, v + 1);
    step(Slot<2>{}, v + 2);
  }
  if (v < n) step(Slot<0>{}, v);
  if (v + 1 < n) step(Slot<1>{}, v + 1);
}

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

// ---- QK^T on the int8 matrix cores (wave 0 of the two-wave kernel).
//
// A field value f of L-level codes (f = c0 + L c1 + L^2 c2) gives the
// features f, F1 = floor(f / L), F2 = floor(f / L^2), and the digits are
// linear in them: c0 = f - L F1, c1 = F1 - L F2, c2 = F2.  So the query's part
// of a field, q_a c0 + q_b c1 + q_c c2, equals
//   q_a f + (q_b - L q_a) F1 + (q_c - L q_b) F2,
// a dot product of small non-negative integers (the features) with a
// transformed query.  The query of each head is first put on a fixed-point
// grid, qint = rint(q 2^S) with |qint| < 2^27 (S from the head's largest
// component; the grid step is 2^-27 of it), so the transformed coefficients
// are exact integers below 2^30.  Each coefficient is split into four signed
// base-256 digits (limbs), and v_mfma_i32_16x16x64_i8 multiplies them with
// the features exactly: A rows are (head, limb) = 16 rows, B columns are 16
// tokens, K runs over 64 feature bytes; the four limb sums of a head are
// recombined per token in fp32.  Integer products need no centring of the
// features, so a feature costs one packed fp16 FMA (the floor trick below) and
// no subtraction.
//
// Layout of one 16-token set: lane (n, kg) = (lane & 15, lane >> 4) holds
// token 4n + s of the tile (s = set) and k-group kg: bytes 12kg .. 12kg+11 of
// a 6-level row (fields 12kg + 0..11), or fields 11kg + 0..10 of a 5-level
// row (a 77-bit window).  Its B bytes per set are, in order:
//   6 levels: F0 of its 12 fields (raw bytes XOR 0x80: f - 128 as int8),
//             then F1 and F2 as fp16 slots 1536 + F (low byte F, high byte
//             0x66), two fields per dword: 15 dwords + 1 zero = 4 MFMAs;
//   5 levels: per group of 4 fields, the slots of f (low byte f < 128), F1
//             and F2: 18 dwords + 2 zeros = 5 MFMAs.
// The A bytes facing a slot's 0x66 byte, a field past the row or a zero dword
// are 0.  The constant -128 of the XORed bytes is added back through the
// MFMA's C input: 128 * sum of the F0 coefficients, in limbs.  The C output
// of lane (n, g) is the four limb sums of head g for token 4n + s.

typedef int i4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i4 mfma_i8(i4 a, i4 b, i4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ i4 as_i4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(i4, make_uint4(a, b, c, d));
}
// Signed base-256 digits of x in [-0x80808080, 0x7F7F7F7F] as four int8
// bytes (lowest digit first): sum_k digit_k 256^k = x.
__device__ __forceinline__ uint32_t limb_bytes(int32_t x) {
  return ((uint32_t)x + 0x80808080u) ^ 0x80808080u;
}
__device__ __forceinline__ uint32_t floor_slots(uint32_t x, int L) {   // see floor_div
  return L == 6 ? __builtin_bit_cast(uint32_t, floor_div<6>(__builtin_bit_cast(h2, x)))
                : __builtin_bit_cast(uint32_t, floor_div<5>(__builtin_bit_cast(h2, x)));
}

constexpr int kCoefSlots = 48;   // per (head, feature): 4 k-groups x 12

// LDS of the query preparation of wave 0 (once per chunk).
struct QPrep {
  int32_t qint[4][kHeadDim + 4];                 // fixed-point queries, 4 zero pads
  uint32_t coef[4][3][kCoefSlots];               // limb bytes of the coefficients
};

template <int L, bool kRot>
__device__ __forceinline__ void qk_wave_i8(const DecodeArgs& a, int seg, int64_t r0, int64_t r1,
                                           int b, int li, int g, const Stage3& st, QPrep& qp) {
  constexpr int R = (L == 6) ? 43 : 38;
  constexpr int NM = (L == 6) ? 4 : 5;          // MFMAs per 16-token set
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, kg = lane >> 4;
  const int layer = a.layer0 + li;
  const int64_t plane_k = (((int64_t)b * a.layers + layer) * a.kv_heads + g) * 2;
  const int cap = (int)a.cap[seg];            // cap * R < 2^31 (checked by the launcher)
  const int ir0 = (int)r0, ir1 = (int)r1;
  const uint8_t* kcodes = a.codes[seg] + plane_k * cap * R;
  const uint8_t* vcodes = kcodes + cap * R;
  const uint32_t* kmg = a.meta[seg] + plane_k * cap;
  const uint32_t bias5 = L == 5 ? bias_register() : 0u;   // 5-level field bias
  const int ntiles = (ir1 - ir0 + kTile - 1) / kTile;

  // byte offset and bit shift of this lane's window within a row, and the
  // dword-aligned offset of set s's window within a tile
  const int kbyte = L == 6 ? 12 * kg : (77 * kg) >> 3;
  const int kbit = L == 6 ? 0 : (77 * kg) & 7;
  int koff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) koff[s] = (4 * n + s) * R + kbyte;

  // Tile v: its V bytes (3 KB from its first row; 16-row byte-planar tiles)
  // -> V buffer S, then this lane's 16-byte windows of its 4 K rows and the
  // K meta of tokens 4n .. 4n+3 -> register slot S.  Past the chunk the
  // buffer ranges are empty (zeros, no memory traffic).
  uint4 kx[3][4], km[3];
  const uint32_t lane16 = 16u * (uint32_t)lane;
  auto issue_v = [&](lds_void* dst, int v) {
    const bool live = v < ntiles;
    const int t0 = ir0 + kTile * v;
    const __amdgpu_buffer_rsrc_t rv = plane_rsrc(vcodes + (live ? t0 * R : 0), live ? (cap - t0) * R : 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dst, 16, (int)lane16, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dst, 16, (int)lane16, 0, 1024, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dst, 16, (int)lane16, 0, 2048, 0);
  };
  auto issue = [&](auto Sc, int v) {
    constexpr int S = decltype(Sc)::value;
    issue_v(lds_at(vbuf_of<S>(st), 0), v);
    const bool live = v < ntiles;
    const int t0 = ir0 + kTile * v;
    const int rows = live ? cap - t0 : 0;
    const int tb = live ? t0 * R : 0;
    const __amdgpu_buffer_rsrc_t rk = plane_rsrc(kcodes + tb, rows * R);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      kx[S][s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, koff[s] & ~3, 0, 0));
    km[S] = __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(plane_rsrc(kmg + (live ? t0 : 0), rows * 4), 16 * n, 0, 0));
  };
  // the queries (dimensions 2 lane, 2 lane + 1 of the 4 heads) are loaded
  // before the first tiles, so that waiting for them drains nothing else
  const uint32_t* qg = reinterpret_cast<const uint32_t*>(a.q) +
                       (((int64_t)b * a.nl + li) * a.q_heads + g * 4) * (kHeadDim / 2);
  uint32_t qw[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) qw[h] = qg[h * (kHeadDim / 2) + lane];
  issue(Slot<0>{}, 0);
  issue(Slot<1>{}, 1);

  // ---- queries (once per chunk, while the first tiles are in flight)
  float cA, cB;                       // this lane's head (kg): logit = cA s_K z + cB m_K
  {
    const float sm = a.sm_scale * kLog2e;   // logits in log2 units
    float cA4[4], cB4[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float y0 = h2f((uint16_t)(qw[h] & 0xFFFFu)), y1 = h2f((uint16_t)(qw[h] >> 16));
      if constexpr (kRot) {
        // rotated cache: q -> H q in fp32 (index bit 0 within the lane,
        // bits 1-6 across lanes)
        constexpr float kNorm = 0.08838834764831845f;   // 1/sqrt(128)
        float u0 = y0 + y1, u1 = y0 - y1;
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
          const float p0 = __shfl_xor(u0, m, 64), p1 = __shfl_xor(u1, m, 64);
          const bool upper = (lane & m) != 0;
          u0 = upper ? p0 - u0 : u0 + p0;
          u1 = upper ? p1 - u1 : u1 + p1;
        }
        y0 = u0 * kNorm;
        y1 = u1 * kNorm;
      }
      const float mx = wave_max(fmaxf(fabsf(y0), fabsf(y1)));
      const int S = mx > 0.0f ? 26 - ilogbf(mx) : 0;
      qp.qint[h][2 * lane] = (int32_t)rintf(ldexpf(y0, S));
      qp.qint[h][2 * lane + 1] = (int32_t)rintf(ldexpf(y1, S));
      if (lane < 4) qp.qint[h][kHeadDim + lane] = 0;
      cA4[h] = sm * ldexpf(1.0f, -S);
      cB4[h] = sm * wave_sum(y0 + y1);
    }
    cA = kg == 0 ? cA4[0] : kg == 1 ? cA4[1] : kg == 2 ? cA4[2] : cA4[3];
    cB = kg == 0 ? cB4[0] : kg == 1 ? cB4[1] : kg == 2 ? cB4[2] : cB4[3];
  }
  wait_lgkm0();   // the wave's qint writes have landed
  // coefficient limbs: slot kgs * 12 + j of (head, feature) is field 12 kgs + j
  // (6 levels) or 11 kgs + j for j < 11 (5 levels); fields past 42 are 0
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    const int idx = lane + 64 * p;                 // (head, slot), 192 of them
    const int h = idx / kCoefSlots, slot = idx - h * kCoefSlots;
    const int kgs = slot / 12, j = slot - kgs * 12;
    const int f = L == 6 ? slot : (j < 11 ? 11 * kgs + j : 99);
    uint32_t c0 = 0, c1 = 0, c2 = 0;
    if (f < 43) {
      const int qa = qp.qint[h][3 * f], qb = qp.qint[h][3 * f + 1], qc = qp.qint[h][3 * f + 2];
      c0 = limb_bytes(qa);
      c1 = limb_bytes(qb - L * qa);
      c2 = limb_bytes(qc - L * qb);
    }
    qp.coef[h][0][slot] = c0;
    qp.coef[h][1][slot] = c1;
    qp.coef[h][2][slot] = c2;
  }
  wait_lgkm0();
  // A operands: lane (row r = 4 h + k, kg) holds limb k of head h's
  // coefficients for the B bytes of k-group kg, in the same order
  i4 A[NM];
  i4 cinit = {0, 0, 0, 0};
  {
    const int h = n >> 2, k = n & 3;
    const uint32_t kk = (uint32_t)k;
    const uint32_t sel_pair = kk | 0x0C00u | ((4u + kk) << 16) | 0x0C000000u;   // [x.k, 0, y.k, 0]
    const uint32_t sel_lo = kk | ((4u + kk) << 8) | 0x0C0C0000u;                // [x.k, y.k, 0, 0]
    const uint32_t sel_hi = 0x0C0Cu | (kk << 16) | ((4u + kk) << 24);           // [0, 0, x.k, y.k]
    uint32_t w[4 * NM];
    auto row = [&](int type, int j0) {
      return *reinterpret_cast<const uint4*>(&qp.coef[h][type][kg * 12 + j0]);
    };
    if constexpr (L == 6) {
      int f0sum = 0;
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const uint4 c0 = row(0, 4 * q), c1 = row(1, 4 * q), c2 = row(2, 4 * q);
        w[q] = perm(c0.y, c0.x, sel_lo) | perm(c0.w, c0.z, sel_hi);
        f0sum = __builtin_amdgcn_sdot4((int)w[q], 0x01010101, f0sum, false);
        w[3 + 2 * q] = perm(c1.z, c1.x, sel_pair);
        w[4 + 2 * q] = perm(c1.w, c1.y, sel_pair);
        w[9 + 2 * q] = perm(c2.z, c2.x, sel_pair);
        w[10 + 2 * q] = perm(c2.w, c2.y, sel_pair);
      }
      w[15] = 0;
      // the XORed bytes are f - 128: add 128 * sum of the F0 coefficients,
      // limb by limb, through the C input (rows 4 g .. 4 g + 3 of lane (n, g))
      f0sum += __shfl_xor(f0sum, 16, 64);
      f0sum += __shfl_xor(f0sum, 32, 64);
#pragma unroll
      for (int i = 0; i < 4; ++i) cinit[i] = 128 * __shfl(f0sum, 4 * kg + i, 64);
    } else {
#pragma unroll
      for (int gi = 0; gi < 3; ++gi) {
        const uint4 c0 = row(0, 4 * gi), c1 = row(1, 4 * gi), c2 = row(2, 4 * gi);
        w[6 * gi + 0] = perm(c0.z, c0.x, sel_pair);
        w[6 * gi + 1] = perm(c0.w, c0.y, sel_pair);
        w[6 * gi + 2] = perm(c1.z, c1.x, sel_pair);
        w[6 * gi + 3] = perm(c1.w, c1.y, sel_pair);
        w[6 * gi + 4] = perm(c2.z, c2.x, sel_pair);
        w[6 * gi + 5] = perm(c2.w, c2.y, sel_pair);
      }
      w[18] = w[19] = 0;
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) A[m] = as_i4(w[4 * m], w[4 * m + 1], w[4 * m + 2], w[4 * m + 3]);
  }

  float frame = -INFINITY;   // this lane's head (kg): kFrameMargin above its running maximum
  auto step = [&](auto Sc, int v) {
    constexpr int S = decltype(Sc)::value;
    const int nt = min(kTile, ir1 - ir0 - kTile * v);
    const uint32_t kmw[4] = {km[S].x, km[S].y, km[S].z, km[S].w};
    float zz[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int t = 4 * n + s;
      const uint32_t x0 = kx[S][s].x, x1 = kx[S][s].y, x2 = kx[S][s].z, x3 = kx[S][s].w;
      uint32_t w[4 * NM];
      if constexpr (L == 6) {
        const int sh = koff[s] & 3;
        const uint32_t d[3] = {__builtin_amdgcn_alignbyte(x1, x0, sh),
                               __builtin_amdgcn_alignbyte(x2, x1, sh),
                               __builtin_amdgcn_alignbyte(x3, x2, sh)};
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          w[q] = d[q] ^ 0x80808080u;
          const uint32_t e = perm(kBias, d[q], 0x04020400u);   // fields 4q, 4q+2 -> slots
          const uint32_t o = perm(kBias, d[q], 0x04030401u);   // fields 4q+1, 4q+3
          const uint32_t e1 = floor_slots(e, 6), o1 = floor_slots(o, 6);
          w[3 + 2 * q] = e1;
          w[4 + 2 * q] = o1;
          w[9 + 2 * q] = floor_slots(e1, 6);
          w[10 + 2 * q] = floor_slots(o1, 6);
        }
        w[15] = 0;
      } else {
        const int bs = 8 * (koff[s] & 3) + kbit;                 // < 32
        const uint32_t w0 = __builtin_amdgcn_alignbit(x1, x0, bs);
        const uint32_t w1 = __builtin_amdgcn_alignbit(x2, x1, bs);
        const uint32_t w2 = __builtin_amdgcn_alignbit(x3, x2, bs);
        const uint32_t G[3] = {w0, __builtin_amdgcn_alignbit(w1, w0, 28),
                               __builtin_amdgcn_alignbit(w2, w1, 24)};
#pragma unroll
        for (int gi = 0; gi < 3; ++gi) {
          uint32_t pa, pb;
          field_pairs(G[gi], pa, pb, bias5);
          const uint32_t a1 = floor_slots(pa, 5), b1 = floor_slots(pb, 5);
          w[6 * gi + 0] = pa;
          w[6 * gi + 1] = pb;
          w[6 * gi + 2] = a1;
          w[6 * gi + 3] = b1;
          w[6 * gi + 4] = floor_slots(a1, 5);
          w[6 * gi + 5] = floor_slots(b1, 5);
        }
        w[18] = w[19] = 0;
      }
      i4 acc = cinit;
#pragma unroll
      for (int m = 0; m < NM; ++m)
        acc = mfma_i8(A[m], as_i4(w[4 * m], w[4 * m + 1], w[4 * m + 2], w[4 * m + 3]), acc);
      // limb sums of head kg -> the integer dot product in fp32
      const int32_t tlo = (acc[1] << 8) + acc[0];
      const int32_t thi = (acc[3] << 8) + acc[2];
      const float zf = fmaf((float)thi, 65536.0f, (float)tlo);
      const float sK = h2f((uint16_t)(kmw[s] & 0xFFFFu));
      const float mK = h2f((uint16_t)(kmw[s] >> 16));
      zz[s] = t < nt ? fmaf(sK * cA, zf, mK * cB) : -INFINITY;   // rows past the chunk: no weight
      __builtin_amdgcn_sched_barrier(0);   // one set's temporaries live at a time
    }
    float* zb = zbuf_of<S>(st);
    *reinterpret_cast<float4*>(zb + kg * kTile + 4 * n) = make_float4(zz[0], zz[1], zz[2], zz[3]);
    // softmax frame of head kg, kFrameMargin above the running maximum; it is
    // raised only when a logit exceeds it (in practice on the first tile)
    const float zmax = fmaxf(fmaxf(zz[0], zz[1]), fmaxf(zz[2], zz[3]));
    if (__ballot(zmax > frame) != 0ull) {
      float m = zmax;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      frame = fmaxf(frame, m + kFrameMargin * kLog2e);
    }
    if (n == 0) zb[4 * kTile + kg] = frame;
    wait_lgkm0();  // logits written
    tile_barrier();
    issue(Slot<(S + 2) % 3>{}, v + 2);   // wave 1 is done with that V buffer
  };
  for_tiles(ntiles, step);
}

template <int L>
__device__ __forceinline__ void pv_wave(const DecodeArgs& a, int seg, int64_t r0, int64_t r1, int b, int li,
                        int g, int64_t u, const Stage3& st) {
  constexpr int R = (L == 6) ? 43 : 38;
  const int lane = threadIdx.x & 63;
  _Float16* wbuf = st.w;
  const int layer = a.layer0 + li;
  const int64_t plane_k = (((int64_t)b * a.layers + layer) * a.kv_heads + g) * 2;
  const int cap = (int)a.cap[seg];            // cap * R < 2^31 (checked by the launcher)
  const int ir0 = (int)r0, ir1 = (int)r1;
  const uint32_t* vmg = a.meta[seg] + (plane_k + 1) * cap;
  const int ntiles = (ir1 - ir0 + kTile - 1) / kTile;

  // Chunk exponent E: w = p * scale_V * 2^E (p <= 1) stays below 2^15, so
  // that the fp16 hi/lo split of w neither overflows nor goes subnormal
  // for the largest weights.  It is set from the first tile's largest V
  // scale and lowered (rescaling what was accumulated) when a later tile
  // holds a scale it cannot take.
  int E = 0;
  float two_e = 1.0f;
  uint32_t slim = 0;        // fp16 bits of the first scale E cannot take (0: E not set yet)

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

  // the lane's V meta word of tile v -> register slot S (wave 0 loads the
  // V bytes); past the chunk the range is empty
  uint32_t vmr[3];
  auto fetch = [&](auto Sc, int v) {
    constexpr int S = decltype(Sc)::value;
    const bool live = v < ntiles;
    const int t0 = ir0 + kTile * v;
    vmr[S] = __builtin_amdgcn_raw_buffer_load_b32(
        plane_rsrc(vmg + (live ? t0 : 0), live ? (cap - t0) * 4 : 0), 4 * lane, 0, 0);
  };
  fetch(Slot<0>{}, 0);
  fetch(Slot<1>{}, 1);

  const int col = lane & 15;
  const int quad = lane >> 4;
  // the 0x66 bias bytes of 5-level fields, held in a register so that the
  // mask and the bias go into one AND-OR
  const uint32_t bias5 = L == 5 ? bias_register() : 0u;
  auto step = [&](auto Sc, int v) {
    constexpr int S = decltype(Sc)::value;
    const int nt = min(kTile, ir1 - ir0 - kTile * v);
    fetch(Slot<(S + 2) % 3>{}, v + 2);
    const uint32_t vm = vmr[S];
    // E from the first tile; lowered when a tile holds a scale it cannot
    // take (then the accumulators are rescaled with the frame below)
    const uint32_t sbits = vm & 0xFFFFu;                 // non-negative fp16: ordered as integers
    float efac = 1.0f;
    if (__ballot(sbits >= slim) != 0ull) {
      const uint32_t smax = wave_max_u32(sbits);
      const int E0 = E;
      E = smax != 0 ? 13 - ilogbf(h2f((uint16_t)smax)) : 0;
      two_e = ldexpf(1.0f, E);
      efac = ldexpf(1.0f, E - E0);                       // the sums so far are 0 on the first tile
      const int e = 15 - E;                              // scales must stay below 2^e
      slim = e >= 16 ? 0x7C00u : e >= -14 ? (uint32_t)(e + 15) << 10 : e >= -24 ? 1u << (e + 24) : 1u;
    }
    tile_barrier();                                      // logits and V bytes of this tile are in LDS
    const float* zb = zbuf_of<S>(st);
    float z[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) z[h] = zb[h * kTile + lane];
    const float4 fr = *reinterpret_cast<const float4*>(zb + 4 * kTile);   // all lanes alike

    // the weights are taken against the frame of wave 0; when it was raised
    // (in practice only on the first tile) what was accumulated is rescaled
    if (fr.x != mref[0] || fr.y != mref[1] || fr.z != mref[2] || fr.w != mref[3] || efac != 1.0f) {
      const float nf[4] = {fr.x, fr.y, fr.z, fr.w};
      float fac[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float ff = mref[h] == nf[h] ? 1.0f : __builtin_amdgcn_exp2f(mref[h] - nf[h]);   // 2^-inf = 0 on the first tile
        mref[h] = nf[h];
        lsum[h] *= ff;
        msum[h] *= ff;
        fac[h] = ff * efac;
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
    const uint8_t* vbuf = vbuf_of<S>(st);
#pragma unroll
    for (int G = 0; G < 2; ++G) {
      if (32 * G >= nt) break;
      // A rows 0-3: w_hi of the 4 heads, rows 4-7: w_lo; rows 8-15 repeat
      // them and only feed C rows 8-15, which are never read.
      const h8 aw = *reinterpret_cast<const h8*>(wbuf + (col & 7) * kTile + 32 * G + 8 * quad);
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
  for_tiles(ntiles, step);   // the tile sequence of wave 0
  write_partial<L>(a, u, lane, E, acc, mref, lsum, msum, kLn2);
}

template <bool kRot>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(4, 8))) void decode_mfma2_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t v0[kBuf], v1[kBuf], v2[kBuf];
  __shared__ __attribute__((aligned(16))) float z0[4 * kTile + 4], z1[4 * kTile + 4], z2[4 * kTile + 4];
  __shared__ __attribute__((aligned(16))) _Float16 w[2 * 4 * kTile];
  __shared__ __attribute__((aligned(16))) QPrep qp;
  Stage3 st;
  st.v0 = v0;
  st.v1 = v1;
  st.v2 = v2;
  st.z0 = z0;
  st.z1 = z1;
  st.z2 = z2;
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
    if (wave == 0) qk_wave_i8<6, kRot>(a, seg, r0, r1, b, li, g, st, qp);
    else pv_wave<6>(a, seg, r0, r1, b, li, g, u, st);
  } else {
    if (wave == 0) qk_wave_i8<5, kRot>(a, seg, r0, r1, b, li, g, st, qp);
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
