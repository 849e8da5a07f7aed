#pragma once
// Device code of the matrix-core decode (see decode_mfma.hip for the
// launchers): included by the translation units that instantiate its
// level pairs, each of which gets its own copy (internal linkage).
// Matrix-core decode attention over pools of 3-, 4-, 5-, 6-, 8- and 16-level rows
// (the SemKV page's mixed-precision cache, Fig. 1 and Table 2: one level
// count per token, the operating pair b_high/b_low = log2 6 / log2 5; the
// cliff study of Fig. 3 adds the neighbouring level counts, and Fig. 18's
// operating point mixes 4 and 3 levels).  Same split-K
// contract as the generic kernel in decode.hip: one workgroup per chunk of
// one pool plane pair (K and V of one sequence, layer and KV head) for the 4
// query heads of the KV head, writing (m, l, o[128]) partials per head.
//
// Both products run on the int8 matrix cores (v_mfma_i32_16x16x64_i8) with
// exact integer sums:
//  * QK^T: the B operand holds small non-negative integer features of the
//    packed K codes (the digits themselves, or for base-L fields the values
//    f, floor(f/L), floor(f/L^2), which the digits are linear in); the A
//    operand holds a fixed-point query, transformed to those features, in
//    four signed byte limbs (rows = head x limb).  The four limb sums of a
//    head are recombined per token in fp32.
//  * PV: the A operand holds the softmax weights w = p * scale_V as 31-bit
//    fixed-point numbers in four signed byte limbs (rows = head x limb, K =
//    the 64 tokens of a tile); the B operand holds the same kind of integer
//    features of the V codes, one column per feature.  The int32 sums are
//    exact; they are recombined in int64, turned into digit sums and moved to
//    fp32 totals only when the weight scale or the softmax frame changes (in
//    practice on the first tile) and at the end of the chunk.
//
// Two waves per chunk.  Wave 0 streams K, computes the logits, the softmax
// weights (against a per-head frame a margin above the running maximum) and
// their limbs; wave 1 streams nothing of its own and runs the PV products.
// A tile's weight limbs and its V bytes pass through LDS with one barrier per
// tile.
#include <utility>

#include "semkv_internal.h"

namespace semkv {
namespace {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef int i4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;
constexpr int kPartialStride = 2 + kHeadDim;
constexpr float kFrameMargin = 8.0f; // softmax frame above the running max (natural log)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kWeightLimit = 1073741824.0f;   // 2^30: fixed-point weights stay below it

// Per level count: packed row bytes R, QK MFMAs per 16-token set (NM), PV
// column sets of 16 fields (PS) and features per field (PF: PV MFMAs per
// set).  Fields are the base-L groups of the row format: 5 codes (a byte)
// for 3 levels, 3 codes for 5 and 6, 4 (a byte of 2-bit codes) for 4, 2
// (nibbles) for 16.
template <int L> struct Lv;
template <> struct Lv<3> { static constexpr int R = 26, NM = 5, PS = 2, PF = 5, G = 5; };
// 8 levels: the 3-bit codes are taken in pairs, a "super-field" F = c0 + 8 c1
// of 6 bits (64 per row), with the features F and floor(F / 8).
template <> struct Lv<8> { static constexpr int R = 48, NM = 4, PS = 4, PF = 2, G = 2; };
template <> struct Lv<6> { static constexpr int R = 43, NM = 4, PS = 3, PF = 3, G = 3; };
template <> struct Lv<5> { static constexpr int R = 38, NM = 5, PS = 3, PF = 3, G = 3; };
template <> struct Lv<4> { static constexpr int R = 32, NM = 2, PS = 2, PF = 4, G = 4; };
template <> struct Lv<16> { static constexpr int R = 64, NM = 2, PS = 4, PF = 2, G = 2; };

__device__ __forceinline__ uint32_t u32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ u16x2 v2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }
__device__ __forceinline__ uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel) {
  return __builtin_amdgcn_perm(s0, s1, sel);
}

// Field values of 3, 5 and 6 levels enter as fp16 in [1024, 2048), where
// the spacing is 1: a 16-bit slot 0x6600 | x is the value 1536 + x (x <
// 512).  One packed fp16 FMA then gives 1536 + floor(x / L) exactly:
// RNE((1536 + x) * m + k) with the constants below, checked exhaustively for
// every field value (x < 243 for 3 levels, 216 for 6, 125 for 5) and so also
// for the floors of floors.
constexpr uint32_t kBias = 0x66666666u;   // perm source of the 0x66 high bytes
template <int L> constexpr float floor_m() {
  return L == 6 ? 0.1663818359375f : L == 5 ? 0.1995849609375f : L == 8 ? 0.12469482421875f : 0.33251953125f;
}
template <int L> constexpr float floor_k() {
  return L == 6 ? 1280.0f : L == 5 ? 1229.0f : L == 8 ? 1344.0f : 1025.0f;
}

template <int L>
__device__ __forceinline__ uint32_t floor_slots(uint32_t x) {   // 1536 + x -> 1536 + floor(x / L)
  constexpr _Float16 m = (_Float16)floor_m<L>(), k = (_Float16)floor_k<L>();
  return __builtin_bit_cast(uint32_t,
                            __builtin_elementwise_fma(__builtin_bit_cast(h2, x), (h2){m, m}, (h2){k, k}));
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
// ---- 8 levels: 4 six-bit super-fields in 24 bits of W, at bits 0, 6, 12,
// 18: slots (F0, F2) from the halves (W[0:15], W[12:27]), (F1, F3) six bits
// higher.
__device__ __forceinline__ void field_pairs6(uint32_t W, uint32_t& pa, uint32_t& pb,
                                             uint32_t bias) {
  const uint32_t h = perm(W >> 12, W, 0x05040100u);
  pa = (h & 0x003F003Fu) | bias;                                       // (F0, F2)
  const u16x2 six = {6, 6};
  pb = (u32(v2(h) >> six) & 0x003F003Fu) | bias;                       // (F1, F3)
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
// over the 16 lanes of a k-group (one head)
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
// LDS address of byte `off` of a shared buffer; the offset is added in the
// LDS address space, so the DMA target stays visibly inside its buffer.
__device__ __forceinline__ lds_void* lds_at(uint8_t* p, int off) { return (lds_void*)((lds_u8*)p + off); }

// One workgroup barrier with no memory fence: the LDS writes before it are
// waited for by the caller; outstanding global->LDS prefetches stay in flight.
__device__ __forceinline__ void tile_barrier() { asm volatile("s_barrier" ::: "memory"); }
// Raw buffer resource over `bytes` bytes from `base` (CDNA buffer
// descriptor, stride 0): loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t plane_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
// s_waitcnt through the builtin (not inline asm), so that the compiler's own
// wait insertion knows what has completed (CDNA s_waitcnt immediate: vmcnt in
// bits 3:0 and 15:14, expcnt in 6:4, lgkmcnt in 11:8).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

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
// floor(x + 1/2) for 0 <= x < 2^31 in one instruction (v_cvt_rpi_i32_f32;
// rint and a conversion take two): the weights' nearest fixed-point value,
// with halves rounded up.
__device__ __forceinline__ int32_t round_int(float x) {
  int32_t r;
  asm("v_cvt_rpi_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}
// Exact value of the four limb sums of one C row group: sum_k c[k] 256^k.
__device__ __forceinline__ int64_t limb_value(i4 c) {
  return (int64_t)c[0] + ((int64_t)c[1] << 8) + ((int64_t)c[2] << 16) + ((int64_t)c[3] << 24);
}

// ---- staging.  Two tiles ahead, all issued by wave 0 in this order per
// tile: the V bytes go global->LDS into one of three buffers (read only by
// wave 1), then the K rows and the K and V meta words go straight into
// registers (three register slots).  Loads complete in issue order, so once
// wave 0 has its K rows of tile t (the compiler waits for those registers
// before it uses them), the V bytes of tile t are in LDS too; the barrier
// after the weights hands them to wave 1.  The V buffer of tile t + 2 is the
// one wave 1 finished before it reached the barrier of tile t, so wave 0
// refills it after that barrier.  Tile slots are compile-time constants (the
// loop is unrolled by three), and the loads of a tile past the chunk go
// through an empty buffer range: they read nothing, and every tile issues the
// same instructions.
//
// Weight exchange per tile slot (wave 0 writes, wave 1 reads after the
// barrier): the A operand of the PV products, dword [head][limb][n] = limb of
// the weights of tokens 4n .. 4n+3, then per head the factor by which the
// totals so far are to be scaled (frame change) and the fixed-point exponent
// of the weights.
constexpr int kWBytes = 4 * 4 * 16 * 4;          // A operand of one tile
constexpr int kWSlot = kWBytes + 32;             // + fac[4], G[4]
struct Stage3 {
  uint8_t *v0, *v1, *v2;       // V tiles
  uint8_t *w0, *w1, *w2;       // weight exchange
  uint32_t *m0, *m1, *m2;      // K meta [64], V meta [64] of a tile
};
template <int S> __device__ __forceinline__ uint8_t* vbuf_of(const Stage3& st) {
  return S == 0 ? st.v0 : S == 1 ? st.v1 : st.v2;
}
template <int S> __device__ __forceinline__ uint8_t* wbuf_of(const Stage3& st) {
  return S == 0 ? st.w0 : S == 1 ? st.w1 : st.w2;
}
template <int S> __device__ __forceinline__ uint32_t* mbuf_of(const Stage3& st) {
  return S == 0 ? st.m0 : S == 1 ? st.m1 : st.m2;
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

// The K and V meta words of tokens 4n .. 4n+3 of one tile from its LDS slot
// (K meta at 0, V meta at 256 bytes).  They arrive by global->LDS loads, the
// first ones issued for their tile; loads complete in issue order, so once at
// most kNewer loads are outstanding (those issued after them) they have
// landed.  The wait and the reads are one asm block: the compiler does not
// see these LDS words as written by the loads and would not wait for them.
template <int kNewer>
__device__ __forceinline__ void read_meta(const uint32_t* mb, int n, uint4& km, uint4& vm) {
  const uint32_t addr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint32_t*)mb + 16u * (uint32_t)n;
  asm volatile("s_waitcnt vmcnt(%2)\n\tds_read_b128 %0, %3\n\tds_read_b128 %1, %3 offset:256\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(km), "=&v"(vm)
               : "n"(kNewer), "v"(addr)
               : "memory");
}

// ---- QK^T (wave 0).
//
// The query of each head is first put on a fixed-point grid, qint = rint(q
// 2^S) with |qint| < 2^27 (S from the head's largest component; the grid step
// is 2^-27 of it).  The coefficient of each B byte is an exact integer below
// 2^30, split into four signed base-256 limbs; A rows are (head, limb) = 16
// rows, B columns are 16 tokens, K runs over 64 feature bytes, and the C
// output of lane (n, g) is the four limb sums of head g for one token.
//
// Layout of one 16-token set: lane (n, kg) = (lane & 15, lane >> 4) holds
// token 4n + s of the tile (s = set) and a quarter of its row (k-group kg):
//   6 levels: bytes 12kg .. 12kg+11 (fields 12kg + 0..11).  B bytes: f of its
//             12 fields (raw bytes XOR 0x80: f - 128 as int8), then F1 =
//             floor(f/6) and F2 = floor(f/36) as fp16 slots 1536 + F (low
//             byte F, high byte 0x66), two fields per dword: 15 dwords + 1
//             zero = 4 MFMAs.  A field value f gives the digits c0 = f - 6 F1,
//             c1 = F1 - 6 F2, c2 = F2, so the query's part of a field, qa c0 +
//             qb c1 + qc c2, is qa f + (qb - 6 qa) F1 + (qc - 6 qb) F2.
//   5 levels: fields 11kg + 0..10 (a 77-bit window), per group of 4 fields
//             the slots of f (low byte f < 128), F1 and F2: 18 dwords + 2
//             zeros = 5 MFMAs.
//   4 levels: bytes 8kg .. 8kg+7; B dword (q, i) = digit i of the 4 fields in
//             byte q of the window: 8 dwords = 2 MFMAs, coefficients qint.
//   16 levels: bytes 16kg .. 16kg+15; B dword (q, i) = nibble i of the 4
//             fields of dword q: 8 dwords = 2 MFMAs.
// A bytes facing a slot's 0x66 byte, a field past the row or a zero dword
// are 0.  The constant -128 of the XORed bytes (6 levels) is added back
// through the MFMA's C input: 128 * sum of the F0 coefficients, in limbs.
constexpr int kCoefSlots = 160;   // coefficient words per head

// LDS of the query preparation of wave 0 (once per chunk, in buffers the
// tile loop has not started to use).
struct QInt { int32_t q[4][kHeadDim + 4]; };           // fixed-point queries, 4 zero pads
struct QCoef { uint32_t c[4][kCoefSlots]; };           // limb bytes of the coefficients

// index of the coefficient of feature `type` of field slot `slot`
template <int L> __device__ __forceinline__ int coef_index(int type, int slot) {
  return L == 4 || L == 3 ? type * 32 + slot : L == 16 || L == 8 ? type * 64 + slot : type * 48 + slot;
}

template <int L, bool kRot>
__device__ __forceinline__ void qk_wave(const DecodeArgs& a, int seg, int64_t r0, int64_t r1,
                                        int b, int li, int g, int64_t u, const Stage3& st,
                                        QInt& qi, QCoef& qc, float* fin) {
  using F = Lv<L>;
  constexpr int R = F::R;
  constexpr int NM = F::NM;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, kg = lane >> 4;
  const int layer = a.layer0 + li;
  const int64_t plane_k = (((int64_t)b * a.layers + layer) * a.kv_heads + g) * 2;
  const int cap = (int)a.cap[seg];            // cap * R < 2^31 (checked by the launcher)
  const int ir0 = (int)r0, ir1 = (int)r1;
  const uint8_t* kcodes = a.codes[seg] + plane_k * cap * R;
  const uint8_t* vcodes = kcodes + cap * R;
  const uint32_t* kmg = a.meta[seg] + plane_k * cap;
  const uint32_t* vmg = kmg + cap;
  const uint32_t bias5 = L == 5 || L == 8 ? bias_register() : 0u;   // 5-level field bias
  const int ntiles = (ir1 - ir0 + kTile - 1) / kTile;

  // byte offset and bit shift of this lane's window within a row, and the
  // offset of set s's window within a tile
  const int kbyte = L == 6 || L == 8 ? 12 * kg : L == 5 ? (77 * kg) >> 3 : L == 4 || L == 3 ? 8 * kg : 16 * kg;
  const int kbit = L == 5 ? (77 * kg) & 7 : 0;
  // set s's window: its dword-aligned byte offset in the tile and its shift
  // (bytes for 3 and 6 levels, bits for 5)
  int kaddr[4], kshift[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int o = (4 * n + s) * R + kbyte;
    kaddr[s] = o & ~3;
    kshift[s] = L == 5 ? 8 * (o & 3) + kbit : o & 3;
  }

  // Tile v: its V bytes (64 R bytes from its first row; 16-row byte-planar
  // tiles) -> V buffer S, then this lane's windows of its 4 K rows and the K
  // and V meta of tokens 4n .. 4n+3 -> register slot S.  Past the chunk the
  // buffer ranges are empty (zeros, no memory traffic).
  constexpr int kVLoads = (64 * R + 1023) / 1024;
  static_assert(kVLoads >= 2 && kVLoads <= 4, "V tile of 2 to 4 KB");
  // loads issued after a tile's meta words until its step begins: the rest
  // of that tile (V bytes, 4 K windows) and all of the next one
  constexpr int kMetaNewer = (kVLoads + 4) + (2 + kVLoads + 4);
  uint4 kx[3][4];
  const uint32_t lane16 = 16u * (uint32_t)lane;
  auto issue_v = [&](lds_void* dst, int v) {
    const bool live = v < ntiles;
    const int t0 = ir0 + kTile * v;
    const __amdgpu_buffer_rsrc_t rv = plane_rsrc(vcodes + (live ? t0 * R : 0), live ? (cap - t0) * R : 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dst, 16, (int)lane16, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dst, 16, (int)lane16, 0, 1024, 0);
    if constexpr (kVLoads > 2) __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dst, 16, (int)lane16, 0, 2048, 0);
    if constexpr (kVLoads > 3) __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dst, 16, (int)lane16, 0, 3072, 0);
  };
  auto issue = [&](auto Sc, int v) {
    constexpr int S = decltype(Sc)::value;
    const bool live = v < ntiles;
    const int t0 = ir0 + kTile * v;
    const int rows = live ? cap - t0 : 0;
    // (an immediate offset would move the global address as well as the LDS
    // one, so the V meta goes through its own LDS pointer)
    lds_void* mk = (lds_void*)(__attribute__((address_space(3))) uint32_t*)mbuf_of<S>(st);
    lds_void* mv = (lds_void*)((__attribute__((address_space(3))) uint32_t*)mbuf_of<S>(st) + 64);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(plane_rsrc(kmg + (live ? t0 : 0), rows * 4), mk, 4,
                                             (int)(4u * (uint32_t)lane), 0, 0, 0);
    // (the V meta range ends with the chunk: rows past it read as {0, 0},
    // which keeps their zero weights finite whatever the pool holds there)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(plane_rsrc(vmg + (live ? t0 : 0), live ? 4 * (ir1 - t0) : 0), mv, 4,
                                             (int)(4u * (uint32_t)lane), 0, 0, 0);
    issue_v(lds_at(vbuf_of<S>(st), 0), v);
    const int tb = live ? t0 * R : 0;
    const __amdgpu_buffer_rsrc_t rk = plane_rsrc(kcodes + tb, rows * R);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if constexpr (L == 4) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b64(rk, kaddr[s], 0, 0);   // (8-byte aligned)
        kx[S][s] = make_uint4(x[0], x[1], 0u, 0u);
      } else {
        kx[S][s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, kaddr[s], 0, 0));
      }
    }
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
      qi.q[h][2 * lane] = (int32_t)rintf(ldexpf(y0, S));
      qi.q[h][2 * lane + 1] = (int32_t)rintf(ldexpf(y1, S));
      if (lane < 4) qi.q[h][kHeadDim + lane] = 0;
      cA4[h] = sm * ldexpf(1.0f, -S);
      cB4[h] = sm * wave_sum(y0 + y1);
    }
    cA = kg == 0 ? cA4[0] : kg == 1 ? cA4[1] : kg == 2 ? cA4[2] : cA4[3];
    cB = kg == 0 ? cB4[0] : kg == 1 ? cB4[1] : kg == 2 ? cB4[2] : cB4[3];
  }
  wait_lgkm0();   // the wave's qint writes have landed
  // coefficient limbs per (head, feature type, field slot).  5 and 6 levels:
  // slot kgs * 12 + j is field 12 kgs + j (6 levels) or 11 kgs + j for j < 11
  // (5 levels), fields past 42 are 0; 4 and 16 levels: the digit's dimension.
  constexpr int kSlots = L == 4 || L == 3 ? 32 : L == 16 || L == 8 ? 64 : 48;
#pragma unroll
  for (int p = 0; p < (4 * kSlots) / 64; ++p) {
    const int idx = lane + 64 * p;                 // (head, slot)
    const int h = idx / kSlots, slot = idx - h * kSlots;
    if constexpr (L == 6 || L == 5) {
      const int kgs = slot / 12, j = slot - kgs * 12;
      const int f = L == 6 ? slot : (j < 11 ? 11 * kgs + j : 99);
      uint32_t c0 = 0, c1 = 0, c2 = 0;
      if (f < 43) {
        const int qa = qi.q[h][3 * f], qb = qi.q[h][3 * f + 1], qcc = qi.q[h][3 * f + 2];
        c0 = limb_bytes(qa);
        c1 = limb_bytes(qb - L * qa);
        c2 = limb_bytes(qcc - L * qb);
      }
      qc.c[h][coef_index<L>(0, slot)] = c0;
      qc.c[h][coef_index<L>(1, slot)] = c1;
      qc.c[h][coef_index<L>(2, slot)] = c2;
    } else if constexpr (L == 3) {
      // field f (byte f) = codes 5f .. 5f+4: coefficient of F_0 = f is q_0,
      // of F_i = floor(f / 3^i) is q_i - 3 q_{i-1}; fields past 25 are 0
      const int* qf = &qi.q[h][5 * min(slot, 25)];
#pragma unroll
      for (int i = 0; i < 5; ++i)
        qc.c[h][coef_index<3>(i, slot)] = slot < 26 ? limb_bytes(i == 0 ? qf[0] : qf[i] - 3 * qf[i - 1]) : 0u;
    } else if constexpr (L == 8) {
      // super-field m = codes 2m, 2m+1: coefficient of F is q_2m, of
      // floor(F / 8) is q_2m+1 - 8 q_2m
      const int qa = qi.q[h][2 * slot], qb = qi.q[h][2 * slot + 1];
      qc.c[h][coef_index<8>(0, slot)] = limb_bytes(qa);
      qc.c[h][coef_index<8>(1, slot)] = limb_bytes(qb - 8 * qa);
    } else {
#pragma unroll
      for (int i = 0; i < Lv<L>::G; ++i)
        qc.c[h][coef_index<L>(i, slot)] = limb_bytes(qi.q[h][Lv<L>::G * slot + i]);
    }
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
    auto row = [&](int type, int s0) {
      return *reinterpret_cast<const uint4*>(&qc.c[h][coef_index<L>(type, s0)]);
    };
    auto pick4 = [&](uint4 c) { return perm(c.y, c.x, sel_lo) | perm(c.w, c.z, sel_hi); };
    if constexpr (L == 6) {
      int f0sum = 0;
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const uint4 c0 = row(0, kg * 12 + 4 * q), c1 = row(1, kg * 12 + 4 * q), c2 = row(2, kg * 12 + 4 * q);
        w[q] = pick4(c0);
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
    } else if constexpr (L == 5) {
#pragma unroll
      for (int gi = 0; gi < 3; ++gi) {
        const uint4 c0 = row(0, kg * 12 + 4 * gi), c1 = row(1, kg * 12 + 4 * gi), c2 = row(2, kg * 12 + 4 * gi);
        w[6 * gi + 0] = perm(c0.z, c0.x, sel_pair);
        w[6 * gi + 1] = perm(c0.w, c0.y, sel_pair);
        w[6 * gi + 2] = perm(c1.z, c1.x, sel_pair);
        w[6 * gi + 3] = perm(c1.w, c1.y, sel_pair);
        w[6 * gi + 4] = perm(c2.z, c2.x, sel_pair);
        w[6 * gi + 5] = perm(c2.w, c2.y, sel_pair);
      }
      w[18] = w[19] = 0;
    } else if constexpr (L == 8) {
      // per group of 4 super-fields (16 kg + 4 gi ..): slots of F for (0, 2),
      // (1, 3), then of floor(F / 8) for the same
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const uint4 c0 = row(0, 16 * kg + 4 * gi), c1 = row(1, 16 * kg + 4 * gi);
        w[4 * gi + 0] = perm(c0.z, c0.x, sel_pair);
        w[4 * gi + 1] = perm(c0.w, c0.y, sel_pair);
        w[4 * gi + 2] = perm(c1.z, c1.x, sel_pair);
        w[4 * gi + 3] = perm(c1.w, c1.y, sel_pair);
      }
    } else if constexpr (L == 3) {
      // f of fields 8kg .. 8kg+7 (XORed bytes), then F_1 .. F_4 as slots:
      // (fields 0, 2), (1, 3), (4, 6), (5, 7) of the window
      int f0sum = 0;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        w[q] = pick4(row(0, 8 * kg + 4 * q));
        f0sum = __builtin_amdgcn_sdot4((int)w[q], 0x01010101, f0sum, false);
#pragma unroll
        for (int i = 1; i < 5; ++i) {
          const uint4 c = row(i, 8 * kg + 4 * q);
          w[2 + 4 * (i - 1) + 2 * q] = perm(c.z, c.x, sel_pair);
          w[3 + 4 * (i - 1) + 2 * q] = perm(c.w, c.y, sel_pair);
        }
      }
      w[18] = w[19] = 0;
      f0sum += __shfl_xor(f0sum, 16, 64);
      f0sum += __shfl_xor(f0sum, 32, 64);
#pragma unroll
      for (int i = 0; i < 4; ++i) cinit[i] = 128 * __shfl(f0sum, 4 * kg + i, 64);
    } else if constexpr (L == 4) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) w[4 * q + i] = pick4(row(i, 8 * kg + 4 * q));
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 2; ++i) w[2 * q + i] = pick4(row(i, 16 * kg + 4 * q));
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) A[m] = as_i4(w[4 * m], w[4 * m + 1], w[4 * m + 2], w[4 * m + 3]);
  }

  // ---- softmax state of this lane's head (kg), partial sums over its tokens
  float frame = -INFINITY;   // kFrameMargin above the running maximum (log2 units)
  int G = 0;                 // fixed-point exponent: w = rint(p scale_V 2^G)
  bool gset = false;
  // The logits are formed as zz = z - bias, with bias = frame - G once the
  // frame is finite, so that 2^zz is p 2^G itself (no subtraction and no
  // scaling per token); thr = frame - bias is the frame in the same terms.
  float bias = 0.0f, thr = -INFINITY;
  float lsum = 0.0f, msum = 0.0f;   // sums of p 2^G and p 2^G min_V

  auto step = [&](auto Sc, int v) {
    constexpr int S = decltype(Sc)::value;
    const int nt = min(kTile, ir1 - ir0 - kTile * v);
    uint4 km, vm;
    read_meta<kMetaNewer>(mbuf_of<S>(st), n, km, vm);
    const uint32_t kmw[4] = {km.x, km.y, km.z, km.w};
    const uint32_t vmw[4] = {vm.x, vm.y, vm.z, vm.w};
    float zz[4];
    i4 accp;
    // limb sums of head kg -> the integer dot product in fp32 -> the logit
    // (log2 units) with the row's K scale and minimum, less the bias
    auto logit = [&](i4 c, uint32_t km) {
      const int32_t tlo = (c[1] << 8) + c[0];
      const int32_t thi = (c[3] << 8) + c[2];
      const float zf = fmaf((float)thi, 65536.0f, (float)tlo);
      const h2 sm = __builtin_bit_cast(h2, km);          // {scale, min}
      return fmaf((float)sm[0], cA * zf, fmaf((float)sm[1], cB, -bias));
    };
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t x0 = kx[S][s].x, x1 = kx[S][s].y, x2 = kx[S][s].z, x3 = kx[S][s].w;
      uint32_t w[4 * NM];
      if constexpr (L == 6) {
        const int sh = kshift[s];
        const uint32_t d[3] = {__builtin_amdgcn_alignbyte(x1, x0, sh),
                               __builtin_amdgcn_alignbyte(x2, x1, sh),
                               __builtin_amdgcn_alignbyte(x3, x2, sh)};
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          w[q] = d[q] ^ 0x80808080u;
          const uint32_t e = perm(kBias, d[q], 0x04020400u);   // fields 4q, 4q+2 -> slots
          const uint32_t o = perm(kBias, d[q], 0x04030401u);   // fields 4q+1, 4q+3
          const uint32_t e1 = floor_slots<6>(e), o1 = floor_slots<6>(o);
          w[3 + 2 * q] = e1;
          w[4 + 2 * q] = o1;
          w[9 + 2 * q] = floor_slots<6>(e1);
          w[10 + 2 * q] = floor_slots<6>(o1);
        }
        w[15] = 0;
      } else if constexpr (L == 5) {
        const int bs = kshift[s];                                // < 32
        const uint32_t w0 = __builtin_amdgcn_alignbit(x1, x0, bs);
        const uint32_t w1 = __builtin_amdgcn_alignbit(x2, x1, bs);
        const uint32_t w2 = __builtin_amdgcn_alignbit(x3, x2, bs);
        const uint32_t Gw[3] = {w0, __builtin_amdgcn_alignbit(w1, w0, 28),
                                __builtin_amdgcn_alignbit(w2, w1, 24)};
#pragma unroll
        for (int gi = 0; gi < 3; ++gi) {
          uint32_t pa, pb;
          field_pairs(Gw[gi], pa, pb, bias5);
          const uint32_t a1 = floor_slots<5>(pa), b1 = floor_slots<5>(pb);
          w[6 * gi + 0] = pa;
          w[6 * gi + 1] = pb;
          w[6 * gi + 2] = a1;
          w[6 * gi + 3] = b1;
          w[6 * gi + 4] = floor_slots<5>(a1);
          w[6 * gi + 5] = floor_slots<5>(b1);
        }
        w[18] = w[19] = 0;
      } else if constexpr (L == 8) {
        // bytes 12 kg .. 12 kg + 11 of the row (4-byte aligned): super-fields
        // 16 kg .. 16 kg + 15 in four 24-bit groups
        const uint32_t Gw[4] = {x0, __builtin_amdgcn_alignbit(x1, x0, 24), __builtin_amdgcn_alignbit(x2, x1, 16),
                                x2 >> 8};
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          uint32_t pa, pb;
          field_pairs6(Gw[gi], pa, pb, bias5);
          w[4 * gi + 0] = pa;
          w[4 * gi + 1] = pb;
          w[4 * gi + 2] = floor_slots<8>(pa);
          w[4 * gi + 3] = floor_slots<8>(pb);
        }
      } else if constexpr (L == 3) {
        const int sh = kshift[s];
        const uint32_t d[2] = {__builtin_amdgcn_alignbyte(x1, x0, sh), __builtin_amdgcn_alignbyte(x2, x1, sh)};
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          w[q] = d[q] ^ 0x80808080u;
          uint32_t e = perm(kBias, d[q], 0x04020400u);   // fields 4q, 4q+2 -> slots
          uint32_t o = perm(kBias, d[q], 0x04030401u);   // fields 4q+1, 4q+3
#pragma unroll
          for (int i = 1; i < 5; ++i) {
            e = floor_slots<3>(e);
            o = floor_slots<3>(o);
            w[2 + 4 * (i - 1) + 2 * q] = e;
            w[3 + 4 * (i - 1) + 2 * q] = o;
          }
        }
        w[18] = w[19] = 0;
      } else if constexpr (L == 4) {
        const uint32_t xs[2] = {x0, x1};
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) w[4 * q + i] = (xs[q] >> (2 * i)) & 0x03030303u;
      } else {
        const uint32_t xs[4] = {x0, x1, x2, x3};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          w[2 * q] = xs[q] & 0x0F0F0F0Fu;
          w[2 * q + 1] = (xs[q] >> 4) & 0x0F0F0F0Fu;
        }
      }
      i4 acc = cinit;
#pragma unroll
      for (int m = 0; m < NM; ++m)
        acc = mfma_i8(A[m], as_i4(w[4 * m], w[4 * m + 1], w[4 * m + 2], w[4 * m + 3]), acc);
      // the logits of the previous set are formed while this set's products
      // run on the matrix core
      if (s > 0) zz[s - 1] = logit(accp, kmw[s - 1]);
      accp = acc;
      __builtin_amdgcn_sched_barrier(0);   // one set's temporaries live at a time
    }
    zz[3] = logit(accp, kmw[3]);
    if (nt < kTile) {                      // rows past the chunk: no weight
#pragma unroll
      for (int s = 0; s < 4; ++s) zz[s] = 4 * n + s < nt ? zz[s] : -INFINITY;
    }
    // softmax frame of head kg, kFrameMargin above the running maximum; it is
    // raised only when a logit exceeds it (in practice on the first tile),
    // and what was summed so far is then scaled by fac
    float fac = 1.0f;
    const float zmax = fmaxf(fmaxf(zz[0], zz[1]), fmaxf(zz[2], zz[3]));
    if (__ballot(zmax > thr) != 0ull) {
      const float nf = fmaxf(frame, (group_max(zmax) + bias) + kFrameMargin * kLog2e);
      fac = nf == frame ? 1.0f : __builtin_amdgcn_exp2f(frame - nf);   // 2^-inf = 0 on the first tile
      // a raised frame shrinks every weight from here on by fac: the
      // fixed-point exponent is taken afresh from this tile (kept, the later
      // weights would lose as many bits as the frame rose)
      gset = gset && nf == frame;
      frame = nf;
      lsum *= fac;
      msum *= fac;
      // this tile's logits against the new frame, and the bias from here on
      const float corr = (bias - frame) + (float)G;
#pragma unroll
      for (int s = 0; s < 4; ++s) zz[s] += corr;
      bias = frame - (float)G;
      thr = (float)G;
    }
    float wv[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float p = __builtin_amdgcn_exp2f(zz[s]);   // p 2^G; 0 past the chunk
      const h2 sm = __builtin_bit_cast(h2, vmw[s]);   // {scale, min}; {0, 0} past the chunk
      lsum += p;
      msum = fmaf(p, (float)sm[1], msum);
      // (+0 addend: one mixed-precision fma; the product is never negative)
      wv[s] = fmaf((float)sm[0], p, 0.0f);
    }
    // fixed-point exponent of head kg: set from the first nonzero weights
    // (and again after each frame raise) to put the largest at 2^28 .. 2^29,
    // lowered when a weight reaches 2^30 (each change rescales the sums:
    // wave 1 moves what it has summed to its totals first)
    const float wmx = fmaxf(fmaxf(wv[0], wv[1]), fmaxf(wv[2], wv[3]));
    if (__ballot(wmx >= kWeightLimit || (!gset && wmx > 0.0f)) != 0ull) {
      const float gm = group_max(wmx);
      if (gm >= kWeightLimit || (!gset && gm > 0.0f)) {
        // (at most 2^100, so that 2^G stays finite whatever the first weights)
        const int dG = min(28 - ilogbf(gm), 100 - G);
        G += dG;
        gset = true;
#pragma unroll
        for (int s = 0; s < 4; ++s) wv[s] = ldexpf(wv[s], dG);
        lsum = ldexpf(lsum, dG);
        msum = ldexpf(msum, dG);
        bias -= (float)dG;
        thr = (float)G;
      }
    }
    // limbs of the 4 tokens, transposed to one dword per limb (tokens 4n ..
    // 4n+3 in byte order) -> [head kg][limb][n]
    // (rounded to nearest: truncation would bias every weight down, and the
    // many small weights of a diffuse softmax add that bias up)
    const uint32_t W0 = limb_bytes(round_int(wv[0])), W1 = limb_bytes(round_int(wv[1]));
    const uint32_t W2 = limb_bytes(round_int(wv[2])), W3 = limb_bytes(round_int(wv[3]));
    const uint32_t t01l = perm(W1, W0, 0x05010400u), t01h = perm(W1, W0, 0x07030602u);
    const uint32_t t23l = perm(W3, W2, 0x05010400u), t23h = perm(W3, W2, 0x07030602u);
    uint32_t* wb = reinterpret_cast<uint32_t*>(wbuf_of<S>(st));
    wb[(4 * kg + 0) * 16 + n] = perm(t23l, t01l, 0x05040100u);
    wb[(4 * kg + 1) * 16 + n] = perm(t23l, t01l, 0x07060302u);
    wb[(4 * kg + 2) * 16 + n] = perm(t23h, t01h, 0x05040100u);
    wb[(4 * kg + 3) * 16 + n] = perm(t23h, t01h, 0x07060302u);
    if (n == 0) {
      reinterpret_cast<float*>(wb + 256)[kg] = fac;
      reinterpret_cast<int*>(wb + 260)[kg] = G;
    }
    wait_lgkm0();  // weights written
    tile_barrier();
    issue(Slot<(S + 2) % 3>{}, v + 2);   // wave 1 is done with that V buffer
  };
  for_tiles(ntiles, step);

  // per-head sums -> the partial record (m, l) and, for wave 1, sum p min_V
  lsum = ldexpf(group_sum(lsum), -G);
  msum = ldexpf(group_sum(msum), -G);
  if (n == 0) {
    float* wsu = a.ws + u * 4 * kPartialStride + kg * kPartialStride;
    wsu[0] = frame * kLn2;   // natural-log units
    wsu[1] = lsum;
    fin[kg] = msum;
  }
  wait_lgkm0();
  tile_barrier();
}

// ---- PV (wave 1).  B operand of lane (col, kg') = 16 bytes: one feature of
// field column col for tokens 16kg' .. 16kg'+15, i.e. byte plane j of one
// 16-row group of the V tile (16 bytes at kg' * 16R + 16j).  Features:
//   6 levels: f XOR 0x80, F1 = floor(f/6), F2 = floor(f/36) (the fp16 slot
//             floor, packed back to bytes); the column of field 47 (none) holds
//             ones in its f feature, which gives the weight sum for the XOR
//             correction.  Set s covers fields 16s .. 16s+15.
//   5 levels: f (from the 7-bit window over planes floor(7j/8), +1), F1, F2.
//   4 levels: digit i of field j (byte j) = (byte >> 2i) & 3.
//   16 levels: nibbles.
// C of lane (col, h): rows 4h .. 4h+3 = the limb sums of head h.
template <int L>
__device__ __forceinline__ void pv_wave(const DecodeArgs& a, int64_t r0, int64_t r1, int64_t u,
                                        const Stage3& st, const float* fin) {
  using F = Lv<L>;
  constexpr int R = F::R;
  constexpr int PS = F::PS, PF = F::PF;
  constexpr int NMP = PS * PF;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;   // C: head grp; A/B: k-group grp
  const int ntiles = ((int)r1 - (int)r0 + kTile - 1) / kTile;
  const uint32_t bias5 = L == 5 || L == 8 ? bias_register() : 0u;

  i4 acc[NMP];
  float T[NMP];                 // digit sums so far, against the current frame
#pragma unroll
  for (int m = 0; m < NMP; ++m) {
    acc[m] = (i4){0, 0, 0, 0};
    T[m] = 0.0f;
  }
  int Gw = 0;                   // fixed-point exponent of what acc holds

  // move the exact sums to the fp32 totals: T = (T + digits(acc) 2^-Gw) fac
  auto flush = [&](float fac) {
    int64_t vv[NMP];
#pragma unroll
    for (int m = 0; m < NMP; ++m) vv[m] = limb_value(acc[m]);
    int64_t Wsum = 0;
    if constexpr (L == 6 || L == 3) {
      // weight sum of head grp: the ones column (last set, f feature, column 15)
      const int64_t x = vv[(PS - 1) * PF + 0];
      const int lo = __shfl((int)(uint32_t)x, 16 * grp + 15, 64);
      const int hi = __shfl((int)(x >> 32), 16 * grp + 15, 64);
      Wsum = (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
    }
#pragma unroll
    for (int s = 0; s < PS; ++s) {
      int64_t d[PF];
      if constexpr (L == 6 || L == 5) {
        const int64_t f0 = vv[s * PF] + (L == 6 ? 128 * Wsum : 0);
        d[0] = f0 - L * vv[s * PF + 1];
        d[1] = vv[s * PF + 1] - L * vv[s * PF + 2];
        d[2] = vv[s * PF + 2];
      } else if constexpr (L == 8) {
        d[0] = vv[s * PF] - 8 * vv[s * PF + 1];
        d[1] = vv[s * PF + 1];
      } else if constexpr (L == 3) {
        d[0] = vv[s * PF] + 128 * Wsum - 3 * vv[s * PF + 1];
#pragma unroll
        for (int i = 1; i < 4; ++i) d[i] = vv[s * PF + i] - 3 * vv[s * PF + i + 1];
        d[4] = vv[s * PF + 4];
      } else {
#pragma unroll
        for (int i = 0; i < PF; ++i) d[i] = vv[s * PF + i];
      }
#pragma unroll
      for (int i = 0; i < PF; ++i)
        T[s * PF + i] = (T[s * PF + i] + (float)ldexp((double)d[i], -Gw)) * fac;
    }
#pragma unroll
    for (int m = 0; m < NMP; ++m) acc[m] = (i4){0, 0, 0, 0};
  };

  auto step = [&](auto Sc, int v) {
    constexpr int S = decltype(Sc)::value;
    tile_barrier();                                      // weights and V bytes of this tile are in LDS
    const uint8_t* wb = wbuf_of<S>(st);
    const float fac = reinterpret_cast<const float*>(wb + kWBytes)[grp];
    const int Gn = reinterpret_cast<const int*>(wb + kWBytes + 16)[grp];
    const i4 Aw = *reinterpret_cast<const i4*>(wb + col * 64 + grp * 16);
    if (__ballot(fac != 1.0f || Gn != Gw) != 0ull) {
      flush(fac);
      Gw = Gn;
    }
    const uint8_t* vb = vbuf_of<S>(st) + grp * 16 * R;
    // every LDS read of the tile first, one wait for all of them: plane j of
    // column j (the field's bit window spans planes j0, j0 + 1 for 5 and 8
    // levels)
    constexpr int NR = (L == 5 || L == 8) ? 2 : 1;
    uint4 xr[PS][NR];
#pragma unroll
    for (int s = 0; s < PS; ++s) {
      const int j = 16 * s + col;
      if constexpr (L == 5) {
        const int j0 = (7 * j) >> 3;
        xr[s][0] = *reinterpret_cast<const uint4*>(vb + 16 * j0);
        xr[s][NR - 1] = *reinterpret_cast<const uint4*>(vb + 16 * j0 + 16);
      } else if constexpr (L == 8) {
        const int j0 = (6 * j) >> 3;
        xr[s][0] = *reinterpret_cast<const uint4*>(vb + 16 * j0);
        xr[s][NR - 1] = *reinterpret_cast<const uint4*>(vb + 16 * min(j0 + 1, R - 1));
      } else {
        xr[s][0] = *reinterpret_cast<const uint4*>(vb + 16 * j);
      }
    }
#pragma unroll
    for (int s = 0; s < PS; ++s) {
      const int j = 16 * s + col;
      uint32_t f[PF][4];
      if constexpr (L == 6) {
        const uint4 x = xr[s][0];
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
        const bool ones = j == 47;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t d = xs[q];
          f[0][q] = ones ? 0x01010101u : d ^ 0x80808080u;
          const uint32_t e1 = floor_slots<6>(perm(kBias, d, 0x04020400u));   // tokens 0, 2
          const uint32_t o1 = floor_slots<6>(perm(kBias, d, 0x04030401u));   // tokens 1, 3
          f[1][q] = perm(o1, e1, 0x06020400u);
          f[2][q] = perm(floor_slots<6>(o1), floor_slots<6>(e1), 0x06020400u);
        }
      } else if constexpr (L == 5) {
        const int bit = 7 * j;
        const uint4 x0 = xr[s][0], x1 = xr[s][NR - 1];
        const uint32_t b0[4] = {x0.x, x0.y, x0.z, x0.w}, b1[4] = {x1.x, x1.y, x1.z, x1.w};
        const u16x2 shv = {(unsigned short)(bit & 7), (unsigned short)(bit & 7)};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t p01 = (u32(v2(perm(b1[q], b0[q], 0x05010400u)) >> shv) & 0x007F007Fu) | bias5;
          const uint32_t p23 = (u32(v2(perm(b1[q], b0[q], 0x07030602u)) >> shv) & 0x007F007Fu) | bias5;
          const uint32_t a1 = floor_slots<5>(p01), c1 = floor_slots<5>(p23);
          f[0][q] = perm(p23, p01, 0x06040200u);
          f[1][q] = perm(c1, a1, 0x06040200u);
          f[2][q] = perm(floor_slots<5>(c1), floor_slots<5>(a1), 0x06040200u);
        }
      } else if constexpr (L == 8) {
        // super-field j: bits 6j .. 6j+5 of the row, in byte planes
        // floor(6j/8) and the next (not read past the row: the bits above
        // the field are masked off)
        const int bit = 6 * j;
        const uint4 x0 = xr[s][0], x1 = xr[s][NR - 1];
        const uint32_t b0[4] = {x0.x, x0.y, x0.z, x0.w}, b1[4] = {x1.x, x1.y, x1.z, x1.w};
        const u16x2 shv = {(unsigned short)(bit & 7), (unsigned short)(bit & 7)};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t p01 = (u32(v2(perm(b1[q], b0[q], 0x05010400u)) >> shv) & 0x003F003Fu) | bias5;
          const uint32_t p23 = (u32(v2(perm(b1[q], b0[q], 0x07030602u)) >> shv) & 0x003F003Fu) | bias5;
          f[0][q] = perm(p23, p01, 0x06040200u);
          f[1][q] = perm(floor_slots<8>(p23), floor_slots<8>(p01), 0x06040200u);
        }
      } else if constexpr (L == 3) {
        const uint4 x = xr[s][0];
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
        const bool ones = j == 31;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t d = xs[q];
          f[0][q] = ones ? 0x01010101u : d ^ 0x80808080u;
          uint32_t e = perm(kBias, d, 0x04020400u);   // tokens 0, 2
          uint32_t o = perm(kBias, d, 0x04030401u);   // tokens 1, 3
#pragma unroll
          for (int i = 1; i < 5; ++i) {
            e = floor_slots<3>(e);
            o = floor_slots<3>(o);
            f[i][q] = perm(o, e, 0x06020400u);
          }
        }
      } else if constexpr (L == 4) {
        const uint4 x = xr[s][0];
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) f[i][q] = (xs[q] >> (2 * i)) & 0x03030303u;
      } else {
        const uint4 x = xr[s][0];
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f[0][q] = xs[q] & 0x0F0F0F0Fu;
          f[1][q] = (xs[q] >> 4) & 0x0F0F0F0Fu;
        }
      }
#pragma unroll
      for (int i = 0; i < PF; ++i)
        acc[s * PF + i] = mfma_i8(Aw, as_i4(f[i][0], f[i][1], f[i][2], f[i][3]), acc[s * PF + i]);
    }
  };
  for_tiles(ntiles, step);   // the tile sequence of wave 0
  tile_barrier();            // wave 0's per-head sums are in LDS
  flush(1.0f);
  const float ms = fin[grp];
  float* o = a.ws + u * 4 * kPartialStride + grp * kPartialStride + 2;
#pragma unroll
  for (int s = 0; s < PS; ++s)
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int dim = F::G * (16 * s + col) + i;
      if (dim < kHeadDim) o[dim] = ms + T[s * PF + i];
    }
}

// ---- the fp16 tail of generation (at most 128 rows, one chunk), handled by
// a workgroup of the same launch, so that it runs alongside the pool chunks
// instead of in a launch of its own.  The rows are the unquantized K and V
// (not rotated on a rotated cache).  QK^T on the 16x16x32 f16 matrix core (A
// rows 0-3 = the 4 query heads, B columns = 16 K rows; fp16 products are
// exact, sums fp32); wave w takes the 16-row blocks w, w + 2, w + 4, w + 6.
// The logits go to LDS, one row per thread for the softmax statistics; then
// thread (rs, dg) sums rows rs, rs + 8, ... over dimensions 8 dg .. 8 dg + 7
// for the 4 heads.  The record is the same (m, l, o[128]) per head as the
// pool chunks', m in natural-log units; on a rotated cache o is stored as
// H o, which the merge's rotation returns to o (H H = I).
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
constexpr int kTailRowsMax = 128;

__device__ __forceinline__ void tail_pair(const DecodeArgs& a, int b, int li, int g, int64_t u,
                                          const Stage3& st) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = (int)min((int64_t)kTailRowsMax, seg_rows(a, 2, b));   // the whole tail
  const int layer = a.layer0 + li;
  const int64_t plane_k = (((int64_t)b * a.layers + layer) * a.kv_heads + g) * 2;
  const uint16_t* kt = a.tail_kv + plane_k * a.block * kHeadDim;
  const uint16_t* vt = kt + (int64_t)a.block * kHeadDim;
  float* z = reinterpret_cast<float*>(st.v0);      // [4][128] logits, then weights
  float* part = reinterpret_cast<float*>(st.v1);   // [4][128] wave 1's output sums
  float* red = reinterpret_cast<float*>(st.w0);    // [2 waves][8]: maxima, sums

  // queries as the A operand (row col < 4 = head col), K rows as B; two
  // rounds of two 16-row blocks (so that this path holds no more registers
  // than the pool path of the lightest level pairs)
  const int col = lane & 15, kg = lane >> 4;
  const uint16_t* qh = a.q + (((int64_t)b * a.nl + li) * a.q_heads + g * 4 + min(col, 3)) * kHeadDim;
  uint4 qa[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qa[ks] = col < 4 ? *reinterpret_cast<const uint4*>(qh + 32 * ks + 8 * kg) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int round = 0; round < 2; ++round) {
    uint4 kb[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 16 * (wave + 2 * (2 * round + j)) + col;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kb[j][ks] = r < n ? *reinterpret_cast<const uint4*>(kt + (int64_t)r * kHeadDim + 32 * ks + 8 * kg)
                          : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, qa[ks]),
                                                     __builtin_bit_cast(h8, kb[j][ks]), acc, 0, 0, 0);
      const int r = 16 * (wave + 2 * (2 * round + j)) + col;
      if (kg == 0 && r < n) {
#pragma unroll
        for (int h = 0; h < 4; ++h) z[h * kTailRowsMax + r] = a.sm_scale * acc[h];
      }
    }
  }
  // the V rows of this thread: rows rs + 8 i, dimensions 8 dg .. 8 dg + 7, in
  // four passes of four rows (the first two loaded now)
  const int dg = tid & 15, rs = tid >> 4;
  auto load_v = [&](int pass, uint4 (&vv)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = rs + 8 * (4 * pass + j);
      vv[j] = r < n ? *reinterpret_cast<const uint4*>(vt + (int64_t)r * kHeadDim + 8 * dg)
                    : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  uint4 va[4], vb[4];
  load_v(0, va);
  load_v(1, vb);
  __syncthreads();                                  // logits in LDS

  // softmax statistics per head, one row per thread
  float zr[4], mx[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    zr[h] = tid < n ? z[h * kTailRowsMax + tid] : -INFINITY;
    mx[h] = wave_max(zr[h]);
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < 4; ++h) red[wave * 8 + h] = mx[h];
  }
  __syncthreads();
  float sm[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    mx[h] = fmaxf(red[h], red[8 + h]);
    const float p = tid < n ? __expf(zr[h] - mx[h]) : 0.0f;
    if (tid < n) z[h * kTailRowsMax + tid] = p;
    sm[h] = wave_sum(p);
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < 4; ++h) red[wave * 8 + 4 + h] = sm[h];
  }
  __syncthreads();                                  // weights and sums in LDS

  float acc[4][8];
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
  auto pv_pass = [&](int pass, const uint4 (&vv)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = rs + 8 * (4 * pass + j);
      if (r < n) {
        const uint32_t w4[4] = {vv[j].x, vv[j].y, vv[j].z, vv[j].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const float p = z[h * kTailRowsMax + r];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            acc[h][e] = fmaf(p, h2f((uint16_t)(w4[e >> 1] >> (16 * (e & 1)))), acc[h][e]);
        }
      }
    }
  };
  pv_pass(0, va);
  load_v(2, va);
  pv_pass(1, vb);
  load_v(3, vb);
  pv_pass(2, va);
  pv_pass(3, vb);
  // rows of the wave's 4 row groups (lanes 16 apart), then wave 1 -> wave 0
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[h][e] += __shfl_xor(acc[h][e], 16, 64);
      acc[h][e] += __shfl_xor(acc[h][e], 32, 64);
    }
  if (wave == 1 && lane < 16) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float4* dst = reinterpret_cast<float4*>(part + h * kHeadDim + 8 * dg);
      dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
  }
  __syncthreads();
  if (wave == 0 && lane < 16) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float4* dst = reinterpret_cast<float4*>(part + h * kHeadDim + 8 * dg);
      const float4 o0 = dst[0], o1 = dst[1];
      dst[0] = make_float4(o0.x + acc[h][0], o0.y + acc[h][1], o0.z + acc[h][2], o0.w + acc[h][3]);
      dst[1] = make_float4(o1.x + acc[h][4], o1.y + acc[h][5], o1.z + acc[h][6], o1.w + acc[h][7]);
    }
  }
  __syncthreads();                                  // o[4][128] in LDS
  if (wave == 0) {
    float* wsu = a.ws + u * 4 * kPartialStride;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float o0 = part[h * kHeadDim + lane], o1 = part[h * kHeadDim + lane + 64];   // dims lane, lane + 64
      if (a.rotate) {
        // o -> H o: index bit 6 within the lane, bits 0-5 across lanes
        const float s0 = o0 + o1, s1 = o0 - o1;
        o0 = s0;
        o1 = s1;
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
          const float p0 = __shfl_xor(o0, m, 64), p1 = __shfl_xor(o1, m, 64);
          const bool upper = (lane & m) != 0;
          o0 = upper ? p0 - o0 : o0 + p0;
          o1 = upper ? p1 - o1 : o1 + p1;
        }
        o0 *= 0.08838834764831845f;   // fp32(1/sqrt(128))
        o1 *= 0.08838834764831845f;
      }
      wsu[h * kPartialStride + 2 + lane] = o0;
      wsu[h * kPartialStride + 2 + lane + 64] = o1;
      if (lane == 0) {
        wsu[h * kPartialStride + 0] = mx[h];
        wsu[h * kPartialStride + 1] = red[4 + h] + red[8 + 4 + h];
      }
    }
  }
}

template <int L> constexpr int vbuf_bytes() {
  return ((64 * Lv<L>::R + 1023) / 1024 * 1024) > 3072 ? ((64 * Lv<L>::R + 1023) / 1024 * 1024) : 3072;
}

template <int LA, int LB, bool kRot>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(4, 8))) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int kVB = vbuf_bytes<LA>() > vbuf_bytes<LB>() ? vbuf_bytes<LA>() : vbuf_bytes<LB>();
  static_assert(sizeof(QCoef) <= kVB, "coefficients live in V buffer 2 before its first tile");
  static_assert(sizeof(QInt) <= 3 * kWSlot, "fixed-point queries live in the weight slots before the first tile");
  __shared__ __attribute__((aligned(16))) uint8_t vb0[kVB], vb1[kVB], vb2[kVB];
  __shared__ __attribute__((aligned(16))) uint8_t wx[3 * kWSlot];
  __shared__ __attribute__((aligned(16))) uint32_t mt0[128], mt1[128], mt2[128];
  __shared__ float fin[4];
  Stage3 st;
  st.v0 = vb0;
  st.v1 = vb1;
  st.v2 = vb2;
  st.w0 = wx;
  st.w1 = wx + kWSlot;
  st.w2 = wx + 2 * kWSlot;
  st.m0 = mt0;
  st.m1 = mt1;
  st.m2 = mt2;

  const int x = blockIdx.x;
  const int b = blockIdx.z;
  const int li = blockIdx.y / a.kv_heads;
  const int g = blockIdx.y % a.kv_heads;
  const int64_t u = (((int64_t)b * a.nl + li) * a.kv_heads + g) * a.nchunks + x;
  if (x >= a.nch[0] + a.nch[1]) {                  // the fp16 tail chunk (launched with the pools)
    tail_pair(a, b, li, g, u, st);
    return;
  }
  const int seg = x < a.nch[0] ? 0 : 1;
  const int ch = seg == 0 ? x : x - a.nch[0];
  const int64_t r0 = (int64_t)ch * a.chunk;
  const int64_t r1 = max(r0, min(r0 + (int64_t)a.chunk, seg_rows(a, seg, b)));   // a ragged batch's own rows
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  QInt& qi = *reinterpret_cast<QInt*>(wx);
  QCoef& qc = *reinterpret_cast<QCoef*>(vb2);
  // The PV wave issues first when both are ready: it has less to do per tile
  // than the QK wave, and so is never the one a tile's barrier waits for.
  if (wave == 1) __builtin_amdgcn_s_setprio(1);
  if (seg == 0) {
    if (wave == 0) qk_wave<LA, kRot>(a, 0, r0, r1, b, li, g, u, st, qi, qc, fin);
    else pv_wave<LA>(a, r0, r1, u, st, fin);
  } else {
    if (wave == 0) qk_wave<LB, kRot>(a, 1, r0, r1, b, li, g, u, st, qi, qc, fin);
    else pv_wave<LB>(a, r0, r1, u, st, fin);
  }
}

// Launch of one level pair's kernel.
template <int LA, int LB, bool kRot>
hipError_t launch_mfma(dim3 grid, const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_mfma_kernel<LA, LB, kRot>), grid, dim3(128), 0, stream, a);
  return hipGetLastError();
}

}  // namespace
}  // namespace semkv
