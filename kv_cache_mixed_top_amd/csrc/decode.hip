// Decode attention over the packed mixed-precision cache (SemKV page, Figs.
// 1 and 5: decoding reads the quantized cache; grouped-query attention of the
// backbones in Table 2).
//
// Split-K over tokens: the work of one (sequence, layer, KV head) is cut into
// chunks of `chunk` rows of one segment (high pool, low pool, fp16 tail).
// One workgroup per chunk computes, for every query head of the group,
//   m = max_t z_t,  l = sum_t exp(z_t - m),  o = sum_t exp(z_t - m) v_t
// with z_t = sm_scale * q . k_t, in two passes (keys, then values) so no
// running rescale is needed.  A merge kernel combines the chunks with a
// log-sum-exp reduction.  Packed rows are staged through LDS and dequantized
// on the fly (x = min + code * scale).
//
// This is the generic kernel: any level count, any group size <= 8, VALU
// arithmetic.
#include "semkv_internal.h"

namespace semkv {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;
constexpr int kChunkMax = 1024;
constexpr int kStageBytes = kTile * 256 + 64;
constexpr int kPartialStride = 2 + kHeadDim;   // m, l, o[128]
constexpr float kHadamardScale = 0.08838834764831845f;   // 1/sqrt(128), fp32

__device__ __forceinline__ float block_reduce(float v, float* buf, bool is_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float t = __shfl_xor(v, o, 64);
    v = is_max ? fmaxf(v, t) : v + t;
  }
  __syncthreads();
  if (lane == 0) buf[wave] = v;
  __syncthreads();
  float r = buf[0];
  for (int w = 1; w < kThreads / 64; ++w) r = is_max ? fmaxf(r, buf[w]) : r + buf[w];
  return r;
}

// code d of a packed row whose byte j is at p[j * stride] (LDS): stride 1
// for row-major K planes, 16 for byte-planar V planes
__device__ __forceinline__ uint32_t unpack_code(const uint8_t* p, int stride, int d,
                                                const RowFmt& f, const uint32_t* pw) {
  const int fi = d / f.g;
  const int i = d - fi * f.g;
  const int bo = fi * f.b;
  const int by = bo >> 3;
  uint32_t v = (uint32_t)p[by * stride] | ((uint32_t)p[(by + 1) * stride] << 8) |
               ((uint32_t)p[(by + 2) * stride] << 16);
  v = (v >> (bo & 7)) & ((1u << f.b) - 1u);
  return (v / pw[i]) % (uint32_t)f.L;
}

struct Seg {
  int seg;       // 0 high, 1 low, 2 tail
  int64_t t0, t1;
};

__device__ __forceinline__ Seg find_seg(const DecodeArgs& a, int x, int b) {
  Seg s;
  int ch;
  if (x < a.nch[0]) {
    s.seg = 0; ch = x;
  } else if (x < a.nch[0] + a.nch[1]) {
    s.seg = 1; ch = x - a.nch[0];
  } else {
    s.seg = 2; ch = x - a.nch[0] - a.nch[1];
  }
  const int64_t n = seg_rows(a, s.seg, b);        // a ragged batch's own rows
  s.t0 = (int64_t)ch * a.chunk;
  s.t1 = max(s.t0, min(s.t0 + (int64_t)a.chunk, n));
  return s;
}

// Stage rows [t, t + nt) of one plane (K or V) into LDS.
__device__ void stage_tile(const DecodeArgs& a, const Seg& sg, int b, int layer, int g,
                           int kvsel, int64_t t, int nt, uint8_t* lds, uint32_t* meta_lds) {
  const int tid = threadIdx.x;
  if (sg.seg < 2) {
    const RowFmt f = a.fmt[sg.seg];
    const int64_t plane = (((int64_t)b * a.layers + layer) * a.kv_heads + g) * 2 + kvsel;
    const uint8_t* base = a.codes[sg.seg] + plane * a.cap[sg.seg] * f.R + t * f.R;
    // t * R is a multiple of 4 (t % 64 == 0); V planes are byte-planar in
    // 16-row tiles, so whole tiles are staged
    const int nd = kvsel == 0 ? (nt * f.R + 3) >> 2 : ((nt + 15) >> 4) * 4 * f.R;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(base);
    uint32_t* dst = reinterpret_cast<uint32_t*>(lds);
    for (int i = tid; i < nd; i += kThreads) dst[i] = src[i];
    const uint32_t* msrc = a.meta[sg.seg] + plane * a.cap[sg.seg] + t;
    for (int i = tid; i < nt; i += kThreads) meta_lds[i] = msrc[i];
  } else {
    const int64_t plane = (((int64_t)b * a.layers + layer) * a.kv_heads + g) * 2 + kvsel;
    const uint16_t* base = a.tail_kv + (plane * a.block + t) * kHeadDim;
    const uint4* src = reinterpret_cast<const uint4*>(base);
    uint4* dst = reinterpret_cast<uint4*>(lds);
    for (int i = tid; i < nt * 16; i += kThreads) dst[i] = src[i];
  }
}

__device__ __forceinline__ float row_value(const Seg& sg, const RowFmt& f, const uint8_t* lds,
                                           const uint32_t* meta_lds, int kvsel, int r, int d,
                                           const uint32_t* pw) {
  if (sg.seg == 2) {
    const uint16_t* row = reinterpret_cast<const uint16_t*>(lds) + r * kHeadDim;
    return h2f(row[d]);
  }
  const uint32_t m = meta_lds[r];
  const float s = h2f((uint16_t)(m & 0xFFFFu));
  const float mn = h2f((uint16_t)(m >> 16));
  const uint32_t c = kvsel == 0
                         ? unpack_code(lds + r * f.R, 1, d, f, pw)
                         : unpack_code(lds + (r >> 4) * 16 * f.R + (r & 15), 16, d, f, pw);
  return fmaf((float)c, s, mn);
}

__global__ __launch_bounds__(kThreads) void decode_partials_kernel(DecodeArgs a) {
  __shared__ float qs[kMaxGroup][kHeadDim];
  __shared__ float sc[kMaxGroup][kChunkMax];
  __shared__ __attribute__((aligned(16))) uint8_t stage[kStageBytes];
  __shared__ uint32_t meta_lds[kTile];
  __shared__ float red[kThreads / 64];
  __shared__ float hmax[kMaxGroup], hsum[kMaxGroup];

  const int tid = threadIdx.x;
  const int x = a.x0 + blockIdx.x;
  const int b = blockIdx.z;
  const Seg sg = find_seg(a, x, b);
  const int li = blockIdx.y / a.kv_heads;
  const int g = blockIdx.y % a.kv_heads;
  const int layer = a.layer0 + li;
  const int G = a.group;
  const int nt_chunk = (int)(sg.t1 - sg.t0);
  const RowFmt f = sg.seg < 2 ? a.fmt[sg.seg] : row_fmt(65536);
  uint32_t pw[6];
  pw[0] = 1;
  for (int i = 1; i < 6; ++i) pw[i] = pw[i - 1] * (uint32_t)f.L;

  for (int i = tid; i < G * kHeadDim; i += kThreads) {
    const int h = i / kHeadDim, d = i - h * kHeadDim;
    qs[h][d] = h2f(a.q[(((int64_t)b * a.nl + li) * a.q_heads + g * G + h) * kHeadDim + d]);
  }
  // Rotated cache: the pool rows hold H k and H v, so their logits take the
  // fp32 rotation H q (the fp16 tail rows are not rotated and take q as
  // given).  Wave w rotates heads w, w + 4: dimensions 2 lane, 2 lane + 1 in
  // the lane (index bit 0), bits 1-6 across lanes.
  const bool rot_rows = a.rotate && sg.seg < 2;
  if (rot_rows) {
    __syncthreads();
    const int lane = tid & 63, wave = tid >> 6;
    for (int h = wave; h < G; h += kThreads / 64) {
      float y0 = qs[h][2 * lane] + qs[h][2 * lane + 1];
      float y1 = qs[h][2 * lane] - qs[h][2 * lane + 1];
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const float p0 = __shfl_xor(y0, m, 64), p1 = __shfl_xor(y1, m, 64);
        const bool upper = (lane & m) != 0;
        y0 = upper ? p0 - y0 : y0 + p0;
        y1 = upper ? p1 - y1 : y1 + p1;
      }
      qs[h][2 * lane] = y0 * kHadamardScale;
      qs[h][2 * lane + 1] = y1 * kHadamardScale;
    }
  }

  // ---- pass 1: logits
  const int r = tid >> 2, qq = tid & 3;
  for (int64_t t = sg.t0; t < sg.t1; t += kTile) {
    const int nt = (int)min((int64_t)kTile, sg.t1 - t);
    __syncthreads();
    stage_tile(a, sg, b, layer, g, 0, t, nt, stage, meta_lds);
    __syncthreads();
    float dot[kMaxGroup];
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) dot[h] = 0.f;
    if (r < nt) {
      for (int d = 32 * qq; d < 32 * qq + 32; ++d) {
        const float x = row_value(sg, f, stage, meta_lds, 0, r, d, pw);
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h)
          if (h < G) dot[h] = fmaf(qs[h][d], x, dot[h]);
      }
    }
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      dot[h] += __shfl_xor(dot[h], 1, 64);
      dot[h] += __shfl_xor(dot[h], 2, 64);
    }
    if (r < nt && qq == 0) {
      const int j = (int)(t - sg.t0) + r;
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h)
        if (h < G) sc[h][j] = a.sm_scale * dot[h];
    }
  }
  __syncthreads();

  // ---- softmax statistics per head
  for (int h = 0; h < G; ++h) {
    float mx = -INFINITY;
    for (int j = tid; j < nt_chunk; j += kThreads) mx = fmaxf(mx, sc[h][j]);
    mx = block_reduce(mx, red, true);
    float sum = 0.f;
    for (int j = tid; j < nt_chunk; j += kThreads) {
      const float p = __expf(sc[h][j] - mx);
      sc[h][j] = p;
      sum += p;
    }
    sum = block_reduce(sum, red, false);
    if (tid == 0) {
      hmax[h] = mx;
      hsum[h] = sum;
    }
  }

  // ---- pass 2: values
  const int d = tid & (kHeadDim - 1);
  const int hh = tid >> 7;   // heads hh, hh + 2, ...
  float acc[kMaxGroup / 2];
#pragma unroll
  for (int k = 0; k < kMaxGroup / 2; ++k) acc[k] = 0.f;
  for (int64_t t = sg.t0; t < sg.t1; t += kTile) {
    const int nt = (int)min((int64_t)kTile, sg.t1 - t);
    __syncthreads();
    stage_tile(a, sg, b, layer, g, 1, t, nt, stage, meta_lds);
    __syncthreads();
    const int j0 = (int)(t - sg.t0);
    for (int rr = 0; rr < nt; ++rr) {
      const float x = row_value(sg, f, stage, meta_lds, 1, rr, d, pw);
#pragma unroll
      for (int k = 0; k < kMaxGroup / 2; ++k) {
        const int h = hh + 2 * k;
        if (h < G) acc[k] = fmaf(sc[h][j0 + rr], x, acc[k]);
      }
    }
  }
  __syncthreads();

  const int64_t u = ((((int64_t)b * a.nl + li) * a.kv_heads + g) * a.nchunks + x);
  float* wsu = a.ws + u * G * kPartialStride;
  if (a.rotate && sg.seg == 2) {
    // Tail rows of a rotated cache are not rotated, while the merge rotates
    // the merged output back: store this chunk's output as H o, so that the
    // merge's rotation returns it to o (H H = I).  o goes through LDS (the
    // logit rows are free now); H o is summed with the signs of H.
    float* ob = &sc[0][0];                       // [G][128]
#pragma unroll
    for (int k = 0; k < kMaxGroup / 2; ++k) {
      const int h = hh + 2 * k;
      if (h < G) ob[h * kHeadDim + d] = acc[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMaxGroup / 2; ++k) {
      const int h = hh + 2 * k;
      if (h < G) {
        float y = 0.f;
        for (int j = 0; j < kHeadDim; ++j)
          y += (__popc(d & j) & 1) ? -ob[h * kHeadDim + j] : ob[h * kHeadDim + j];
        acc[k] = y * kHadamardScale;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kMaxGroup / 2; ++k) {
    const int h = hh + 2 * k;
    if (h < G) wsu[h * kPartialStride + 2 + d] = acc[k];
  }
  if (tid < G) {
    wsu[tid * kPartialStride + 0] = hmax[tid];
    wsu[tid * kPartialStride + 1] = hsum[tid];
  }
}

// fp16 tail chunks next to the matrix-core pool kernel (query group of 4).
// The tail holds fewer than `block` <= 1024 rows per (sequence, layer, KV
// head), read once each for K and V: every thread keeps eight independent
// 16-byte loads in flight per 128 rows, and the chunk's logits stay in LDS,
// so the chunk costs a few memory latencies.  It writes the same partial
// record (m, l, o[128]) per query head as the other decode kernels.
constexpr int kTailGroup = 4;
constexpr int kTailRows = 128;     // rows per pass over the chunk
constexpr int kTailMax = 1024;     // rows per chunk, >= block

// The tail chunk's output o[h][d] (the sum of the 4 waves' parts) -> the
// partial record; wave h stores head h, dimensions 2 lane and 2 lane + 1.
// With a rotated cache the tail rows are not rotated (only quantized rows
// are), while the merge rotates the merged output back; the record is then
// stored as H o (fp32 butterflies over d: bit 0 in the lane, bits 1-6 across
// lanes), which that rotation returns to o since H H = I.
static_assert(kThreads == 64 * kTailGroup, "one wave per query head of the group");
__device__ __forceinline__ void store_tail_output(const DecodeArgs& a, float* wsu,
                                                  const float (&part)[kThreads / 64][kTailGroup][kHeadDim],
                                                  int tid) {
  const int h = tid >> 6, lane = tid & 63;
  float y0 = part[0][h][2 * lane] + part[1][h][2 * lane] + part[2][h][2 * lane] + part[3][h][2 * lane];
  float y1 = part[0][h][2 * lane + 1] + part[1][h][2 * lane + 1] + part[2][h][2 * lane + 1] +
             part[3][h][2 * lane + 1];
  if (a.rotate) {
    float s0 = y0 + y1, s1 = y0 - y1;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const float p0 = __shfl_xor(s0, m, 64), p1 = __shfl_xor(s1, m, 64);
      const float sg = (lane & m) ? -1.0f : 1.0f;   // upper lane: partner - own
      s0 = fmaf(s0, sg, p0);
      s1 = fmaf(s1, sg, p1);
    }
    y0 = s0 * kHadamardScale;
    y1 = s1 * kHadamardScale;
  }
  *reinterpret_cast<float2*>(wsu + h * kPartialStride + 2 + 2 * lane) = make_float2(y0, y1);
}

__global__ __launch_bounds__(kThreads) void decode_tail_kernel(DecodeArgs a) {
  __shared__ float qs[kTailGroup][kHeadDim];
  __shared__ float z[kTailGroup][kTailMax];
  __shared__ __attribute__((aligned(16))) float part[kThreads / 64][kTailGroup][kHeadDim];
  __shared__ float red[kThreads / 64][2 * kTailGroup];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int x = a.x0 + blockIdx.x;
  const int ch = x - a.nch[0] - a.nch[1];
  const int64_t t0 = (int64_t)ch * a.chunk;
  const int b = blockIdx.z;
  const int n = (int)max((int64_t)0, min(t0 + (int64_t)a.chunk, seg_rows(a, 2, b)) - t0);
  const int li = blockIdx.y / a.kv_heads;
  const int g = blockIdx.y % a.kv_heads;
  const int layer = a.layer0 + li;
  const int64_t plane_k = (((int64_t)b * a.layers + layer) * a.kv_heads + g) * 2;
  const uint16_t* kt = a.tail_kv + (plane_k * a.block + t0) * kHeadDim;
  const uint16_t* vt = a.tail_kv + ((plane_k + 1) * a.block + t0) * kHeadDim;

  for (int i = tid; i < kTailGroup * kHeadDim; i += kThreads) {
    const int h = i / kHeadDim, d = i - h * kHeadDim;
    qs[h][d] = h2f(a.q[(((int64_t)b * a.nl + li) * a.q_heads + g * kTailGroup + h) * kHeadDim + d]);
  }
  __syncthreads();

  // ---- logits: two threads per row, 64 dimensions each
  {
    const int rr = tid >> 1, half = tid & 1;
    for (int r0 = 0; r0 < n; r0 += kTailRows) {
      const int r = r0 + rr;
      uint4 kv[8];
      if (r < n) {
        const uint4* src = reinterpret_cast<const uint4*>(kt + (int64_t)r * kHeadDim + 64 * half);
#pragma unroll
        for (int i = 0; i < 8; ++i) kv[i] = src[i];
      }
      float dot[kTailGroup] = {0.f, 0.f, 0.f, 0.f};
      if (r < n) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t w4[4] = {kv[i].x, kv[i].y, kv[i].z, kv[i].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float xv = h2f((uint16_t)(w4[e >> 1] >> (16 * (e & 1))));
            const int d = 64 * half + 8 * i + e;
#pragma unroll
            for (int h = 0; h < kTailGroup; ++h) dot[h] = fmaf(qs[h][d], xv, dot[h]);
          }
        }
      }
#pragma unroll
      for (int h = 0; h < kTailGroup; ++h) dot[h] += __shfl_xor(dot[h], 1, 64);
      if (r < n && half == 0) {
#pragma unroll
        for (int h = 0; h < kTailGroup; ++h) z[h][r] = a.sm_scale * dot[h];
      }
    }
  }
  __syncthreads();

  // ---- softmax statistics per head: max, then p = exp(z - max) and the sum
  float mx[kTailGroup], sum[kTailGroup];
#pragma unroll
  for (int h = 0; h < kTailGroup; ++h) {
    float m = -INFINITY;
    for (int r = tid; r < n; r += kThreads) m = fmaxf(m, z[h][r]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    mx[h] = m;
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < kTailGroup; ++h) red[wave][h] = mx[h];
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < kTailGroup; ++h) {
    mx[h] = fmaxf(fmaxf(red[0][h], red[1][h]), fmaxf(red[2][h], red[3][h]));
    float sl = 0.f;
    for (int r = tid; r < n; r += kThreads) {
      const float pr = __expf(z[h][r] - mx[h]);
      z[h][r] = pr;
      sl += pr;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sl += __shfl_xor(sl, o, 64);
    sum[h] = sl;
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < kTailGroup; ++h) red[wave][kTailGroup + h] = sum[h];
  }
  __syncthreads();

  // ---- values: 16 threads per row (8 dimensions each), 16 rows per pass
  const int dg = tid & 15, rs = tid >> 4;
  float acc[kTailGroup][8];
#pragma unroll
  for (int h = 0; h < kTailGroup; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  for (int r0 = 0; r0 < n; r0 += kTailRows) {
    uint4 vv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = r0 + rs + 16 * i;
      if (r < n) vv[i] = reinterpret_cast<const uint4*>(vt + (int64_t)r * kHeadDim)[dg];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = r0 + rs + 16 * i;
      if (r < n) {
        const uint32_t w4[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
        for (int h = 0; h < kTailGroup; ++h) {
          const float pr = z[h][r];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            acc[h][e] = fmaf(pr, h2f((uint16_t)(w4[e >> 1] >> (16 * (e & 1)))), acc[h][e]);
        }
      }
    }
  }
  // rows rs and rs + 4k of a wave share dimensions: reduce over the 4 row
  // groups of the wave, then over the 4 waves through LDS
#pragma unroll
  for (int h = 0; h < kTailGroup; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[h][e] += __shfl_xor(acc[h][e], 16, 64);
      acc[h][e] += __shfl_xor(acc[h][e], 32, 64);
    }
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < kTailGroup; ++h) {
      float4* dst = reinterpret_cast<float4*>(&part[wave][h][8 * dg]);
      dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
  }
  __syncthreads();

  const int64_t u = ((((int64_t)b * a.nl + li) * a.kv_heads + g) * a.nchunks + x);
  float* wsu = a.ws + u * kTailGroup * kPartialStride;
  store_tail_output(a, wsu, part, tid);
  if (tid < kTailGroup) {
    wsu[tid * kPartialStride + 0] = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
    wsu[tid * kPartialStride + 1] = red[0][kTailGroup + tid] + red[1][kTailGroup + tid] +
                                    red[2][kTailGroup + tid] + red[3][kTailGroup + tid];
  }
}

// A tail of at most 128 rows in one chunk runs inside the matrix-core launch
// (decode_mfma_kernel.h); decode_tail_kernel above takes longer tails.
constexpr int kTailSmall = 128;

// Log-sum-exp merge of the chunk partials of one (sequence, layer, query
// head): the chunk maxima and sums are read in parallel, the weights
// exp(m_c - M) go to LDS, then each thread combines one output dimension
// with an unrolled loop over the chunks.
// P chunk groups per workgroup: 4 when a head has many chunks (short
// per-layer launches), 1 otherwise.
template <int P>
__global__ __launch_bounds__(P * kHeadDim) void decode_merge_kernel(DecodeArgs a) {
  constexpr int kMergeParts = P;
  constexpr int kMergeThreads = P * kHeadDim;
  extern __shared__ float wch[];           // nchunks weights
  __shared__ float red[kMergeThreads / 64];
  __shared__ float part[P][kHeadDim];
  const int h = blockIdx.x, li = blockIdx.y, b = blockIdx.z;
  const int G = a.group;
  const int g = h / G, hl = h - g * G;
  const int tid = threadIdx.x;
  const int d = tid & (kHeadDim - 1), pi = tid / kHeadDim;
  const int64_t u0 = (((int64_t)b * a.nl + li) * a.kv_heads + g) * a.nchunks;
  const float* ws = a.ws;
  const int nc = a.nchunks;
  constexpr int kWaves = kMergeThreads / 64;
  float M = -INFINITY;
  for (int c = tid; c < nc; c += kMergeThreads) M = fmaxf(M, ws[((u0 + c) * G + hl) * kPartialStride]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  if ((tid & 63) == 0) red[tid >> 6] = M;
  __syncthreads();
  M = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, red[w]);
  float den = 0.f;
  for (int c = tid; c < nc; c += kMergeThreads) {
    const float* p = ws + ((u0 + c) * G + hl) * kPartialStride;
    const float w = __expf(p[0] - M);
    wch[c] = w;
    den = fmaf(w, p[1], den);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o, 64);
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = den;
  __syncthreads();
  den = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) den += red[w];
  // chunks pi, pi + P, ... of this dimension, eight loads in flight
  float num = 0.f;
  const float* pd = ws + (u0 * G + hl) * kPartialStride + 2 + d;
  const int64_t step = (int64_t)G * kPartialStride;
  int c = pi;
  for (; c + 7 * kMergeParts < nc; c += 8 * kMergeParts) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = pd[(int64_t)(c + e * kMergeParts) * step];
#pragma unroll
    for (int e = 0; e < 8; ++e) num = fmaf(wch[c + e * kMergeParts], v[e], num);
  }
  for (; c + 3 * kMergeParts < nc; c += 4 * kMergeParts) {
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = pd[(int64_t)(c + e * kMergeParts) * step];
#pragma unroll
    for (int e = 0; e < 4; ++e) num = fmaf(wch[c + e * kMergeParts], v[e], num);
  }
  for (; c < nc; c += kMergeParts) num = fmaf(wch[c], pd[(int64_t)c * step], num);
  float* out = a.out + (((int64_t)b * a.nl + li) * a.q_heads + h) * kHeadDim;
  if (P == 1 && !a.rotate) {
    out[d] = num / den;
    return;
  }
  float val = 0.f;
  if (P == 1) {
    val = num / den;
  } else {
    part[pi][d] = num;
    __syncthreads();
    if (pi == 0) {
      num = part[0][d];
#pragma unroll
      for (int k = 1; k < kMergeParts; ++k) num += part[k][d];
      val = num / den;
    }
  }
  if (a.rotate) {
    // rotated cache: the output is rotated back, o -> H o, across the 128
    // threads of chunk group 0 (index bits 0-5 within a wave, bit 6 across
    // the two waves through LDS)
    __shared__ float xch[kHeadDim];
    if (pi == 0) {
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const float p = __shfl_xor(val, m, 64);
        val = (d & m) ? p - val : val + p;
      }
      xch[d] = val;
    }
    __syncthreads();
    if (pi == 0) {
      const float p = xch[d ^ 64];
      val = ((d & 64) ? p - val : val + p) * kHadamardScale;
    }
  }
  if (pi == 0) out[d] = val;
}

// Merge of one (sequence, layer, KV head) with 4 query heads by one wave,
// for up to C chunks: every load is issued before the math, so the merge
// costs about one memory latency.
// Lane c * 4 + h reads (m, l) of chunk c and head h; the per-head maximum
// and sum of weighted l are combined across the lanes of a head; each lane
// then sums dimensions lane and lane + 64 of the 4 heads over the chunks.
// Chunk order and the combination rule match the other merge kernels up to
// the order of the floating-point additions.
template <int C>
__global__ __launch_bounds__(64) void decode_merge_unit_kernel(DecodeArgs a) {
  constexpr int G = 4;
  const int lane = threadIdx.x, h4 = lane & 3, c4 = lane >> 2;
  const int g = blockIdx.x, li = blockIdx.y, b = blockIdx.z;
  const int nc = a.nchunks;
  const int64_t unit = ((int64_t)b * a.nl + li) * a.kv_heads + g;
  const float* base = a.ws + unit * nc * G * kPartialStride;
  // all loads first
  const float* pm = base + ((int64_t)min(c4, nc - 1) * G + h4) * kPartialStride;
  const float m_own = pm[0], l_own = pm[1];
  float ov[C][G][2];
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float* p = base + ((int64_t)min(c, nc - 1) * G + h) * kPartialStride + 2;
      ov[c][h][0] = c < nc ? p[lane] : 0.f;
      ov[c][h][1] = c < nc ? p[lane + 64] : 0.f;
    }
  // per-head maximum and denominator over the chunks (lanes of one head)
  float M = c4 < nc ? m_own : -INFINITY;
#pragma unroll
  for (int o = 4; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  const float w_own = c4 < nc ? __expf(m_own - M) : 0.f;
  float den = w_own * l_own;
#pragma unroll
  for (int o = 4; o < 64; o <<= 1) den += __shfl_xor(den, o, 64);
  float num[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) num[h][0] = num[h][1] = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float w = __shfl(w_own, 4 * c + h, 64);   // 0 for c >= nc
      num[h][0] = fmaf(w, ov[c][h][0], num[h][0]);
      num[h][1] = fmaf(w, ov[c][h][1], num[h][1]);
    }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float d = __shfl(den, h, 64);
    float o0 = num[h][0] / d, o1 = num[h][1] / d;            // dimensions lane, lane + 64
    if (a.rotate) {
      // rotated cache: o -> H o (index bit 6 within the lane, bits 0-5 across lanes)
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
      o0 *= kHadamardScale;
      o1 *= kHadamardScale;
    }
    float* o = a.out + (((int64_t)b * a.nl + li) * a.q_heads + g * G + h) * kHeadDim;
    o[lane] = o0;
    o[lane + 64] = o1;
  }
}

}  // namespace

int decode_chunk_tokens(int64_t tokens_per_unit, int64_t units) {
  const int64_t target_wg = 4096;
  int64_t desired = (target_wg + units - 1) / (units > 0 ? units : 1);
  if (desired < 1) desired = 1;
  int64_t c = (tokens_per_unit + desired - 1) / desired;
  c = (c + kTile - 1) / kTile * kTile;
  if (c < kTile) c = kTile;
  if (c > kChunkMax) c = kChunkMax;
  return (int)c;
}

int64_t decode_partial_floats_per_chunk(int group) { return (int64_t)group * kPartialStride; }

hipError_t launch_decode_generic(const DecodeArgs& a, int count, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  dim3 grid(count, a.nl * a.kv_heads, a.batch);
  hipLaunchKernelGGL(decode_partials_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

bool decode_use_mfma(const DecodeArgs& a) { return decode_mfma_supported(a); }

hipError_t launch_decode_partials(const DecodeArgs& a, hipStream_t stream) {
  DecodeArgs g = a;
  if (decode_use_mfma(a)) {
    // a tail of one chunk of at most 128 rows runs in the pool launch itself
    const bool fold = a.nch[2] == 1 && a.block <= kTailSmall;
    hipError_t e = launch_decode_mfma(a, fold, stream);
    if (e != hipSuccess || fold) return e;
    g.x0 = a.nch[0] + a.nch[1];          // the fp16 tail chunks
    if (a.nch[2] <= 0) return hipSuccess;
    dim3 grid(a.nch[2], a.nl * a.kv_heads, a.batch);
    hipLaunchKernelGGL(decode_tail_kernel, grid, dim3(kThreads), 0, stream, g);
    return hipGetLastError();
  }
  g.x0 = 0;
  return launch_decode_generic(g, a.nchunks, stream);
}

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream) {
  if (a.group == 4 && a.nchunks <= 16) {
    const dim3 ug(a.kv_heads, a.nl, a.batch);
    if (a.nchunks <= 8)
      hipLaunchKernelGGL(decode_merge_unit_kernel<8>, ug, dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL(decode_merge_unit_kernel<16>, ug, dim3(64), 0, stream, a);
    return hipGetLastError();
  }
  dim3 grid(a.q_heads, a.nl, a.batch);
  if (a.nchunks > 32) {
    hipLaunchKernelGGL(decode_merge_kernel<4>, grid, dim3(4 * kHeadDim), a.nchunks * sizeof(float),
                       stream, a);
  } else {
    hipLaunchKernelGGL(decode_merge_kernel<1>, grid, dim3(kHeadDim), a.nchunks * sizeof(float),
                       stream, a);
  }
  return hipGetLastError();
}

int decode_mfma_chunk_rows(int64_t n_high, int64_t n_low, int64_t units) {
  // Chunks fill whole rounds of the resident workgroup slots.  A launch that
  // fits one round with chunks of at most kMfmaChunkExact rows (the longest
  // whose PV limb sums stay exact in int32) takes that one round: every
  // chunk start costs its query preparation, pipeline fill and epilogue, so
  // one round of long chunks beats several of short ones (measured on 128k
  // contexts: 564 us against 595 us).  Otherwise a chunk holds at most
  // kMfmaChunkMax rows and the launch takes several rounds of similar chunks,
  // which the dispatcher balances better than a few long ones.  A chunk
  // holds at least kMfmaChunkMin rows: its fixed work then spreads over four
  // tiles.  (A launch over few (sequence, layer, KV head) units, such as one
  // layer of one sequence, would otherwise take one- or two-tile chunks.)
  constexpr int64_t kMfmaChunkExact = 16384;
  constexpr int64_t kMfmaChunkMax = 4096;
  constexpr int64_t kMfmaChunkMin = 4 * kTile;
  const int64_t slots = decode_mfma_resident_waves();
  int64_t per_round = slots / (units > 0 ? units : 1);
  if (per_round < 2) per_round = 2;
  auto count = [&](int64_t c) { return (n_high + c - 1) / c + (n_low + c - 1) / c; };
  auto fit = [&](int64_t target) {
    int64_t c = (n_high + n_low + target - 1) / target;
    c = (c + kTile - 1) / kTile * kTile;
    if (c < kTile) c = kTile;
    while (count(c) > target) c += kTile;   // smallest tile multiple that fits
    return c;
  };
  int64_t c = fit(per_round);
  const bool one_round = c <= kMfmaChunkExact && units * count(c) <= slots;
  // Several rounds: chunks of at most kMfmaChunkMax rows, or twice that when
  // one pool holds at most an eighth of the rows and the units fit the slots
  // (then the minority pool is one short chunk per unit and the majority
  // pool's chunks are alike, so longer chunks save starts without
  // unbalancing the last round: measured 0.5-18% faster at a fraction of
  // 0.1 or 0.9 over 4 x 32k, and 5-10% slower at 0.25 and 0.75).
  const int64_t minority = n_high < n_low ? n_high : n_low;
  const int64_t cap = units <= slots && minority > 0 && 8 * minority <= n_high + n_low
                          ? 2 * kMfmaChunkMax : kMfmaChunkMax;
  if (c > cap && !one_round) c = fit(per_round * ((c + cap - 1) / cap));
  if (c < kMfmaChunkMin) c = kMfmaChunkMin;
  return (int)c;
}

}  // namespace semkv
