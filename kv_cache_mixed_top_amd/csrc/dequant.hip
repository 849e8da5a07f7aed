// Reconstruction of packed pool rows: x = min + code * scale per value (the
// affine integer-level quantizer of the SemKV page, Table 6, undone), and for
// a Hadamard-rotated cache (Table 2's quantizer with rotation) the row
// rotated back by H.  For inspection and quality measurement; the decode
// kernels never materialise these rows.
//
// One workgroup of 256 threads = 64 rows x 4 lanes per tile of one plane;
// lane q of a row unpacks dimensions 32q .. 32q+31 straight from the packed
// bytes in global memory (K planes row-major, V planes byte-planar in
// 16-row tiles).  Rotated rows go through LDS for the 128-point transform.
#include "semkv_internal.h"

namespace semkv {
namespace {

constexpr int kRowsPerTile = 64;
constexpr int kThreads = 256;
constexpr float kHadamardScale = 0.08838834764831845f;   // fp32(1/sqrt(128))

// Code d of row `row` of a plane starting at `plane` (byte j of the row at
// plane + row*R + j for K, plane + (row/16)*16R + 16j + row%16 for V).
__device__ __forceinline__ uint32_t code_at(const uint8_t* plane, int64_t row, int planar,
                                            const RowFmt& f, int d, const uint32_t* pw) {
  const int fi = d / f.g;
  const int i = d - fi * f.g;
  const int bo = fi * f.b;
  uint32_t v = 0;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int j = (bo >> 3) + k;
    if (j < f.R) {
      const int64_t off = planar ? (row >> 4) * 16 * f.R + 16 * j + (row & 15) : row * f.R + j;
      v |= (uint32_t)plane[off] << (8 * k);
    }
  }
  v = (v >> (bo & 7)) & ((f.b >= 32) ? 0xFFFFFFFFu : ((1u << f.b) - 1u));
  return (v / pw[i]) % (uint32_t)f.L;
}

__global__ __launch_bounds__(kThreads) void dequant_kernel(DequantArgs a) {
  __shared__ float rows[kRowsPerTile][kHeadDim + 1];
  const int tid = threadIdx.x, r = tid >> 2, q = tid & 3;
  const int64_t row = a.row0 + (int64_t)blockIdx.x * kRowsPerTile + r;
  const int pl = blockIdx.y;                       // (b, kv head, K|V) of the layer
  const int kvsel = pl & 1, head = (pl >> 1) % a.kv_heads, b = (pl >> 1) / a.kv_heads;
  const int64_t plane = (((int64_t)b * a.layers + a.layer) * a.kv_heads + head) * 2 + kvsel;
  const RowFmt f = a.fmt;
  const bool valid = row < a.row0 + a.nrows;
  uint32_t pw[6];
  pw[0] = 1;
#pragma unroll
  for (int i = 1; i < 6; ++i) pw[i] = pw[i - 1] * (uint32_t)f.L;
  float x[32];
  if (valid) {
    const uint8_t* base = a.codes + plane * a.cap * f.R;
    const uint32_t m = a.meta[plane * a.cap + row];
    const float s = h2f((uint16_t)(m & 0xFFFFu)), mn = h2f((uint16_t)(m >> 16));
#pragma unroll 4
    for (int e = 0; e < 32; ++e) x[e] = fmaf((float)code_at(base, row, kvsel, f, 32 * q + e, pw), s, mn);
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = 0.f;
  }
  if (a.rotate) {
    // x -> H x over the 128 values of the row: through LDS, each lane sums
    // its 32 outputs with the signs of the normalized Sylvester matrix
#pragma unroll
    for (int e = 0; e < 32; ++e) rows[r][32 * q + e] = x[e];
    __syncthreads();
#pragma unroll 2
    for (int e = 0; e < 32; ++e) {
      const int d = 32 * q + e;
      float y = 0.f;
      for (int j = 0; j < kHeadDim; ++j) y += (__popc(d & j) & 1) ? -rows[r][j] : rows[r][j];
      x[e] = y * kHadamardScale;
    }
  }
  if (valid) {
    float* o = a.out + (((int64_t)b * a.kv_heads + head) * 2 + kvsel) * a.nrows * kHeadDim +
               (row - a.row0) * kHeadDim + 32 * q;
#pragma unroll
    for (int e = 0; e < 32; e += 4)
      *reinterpret_cast<float4*>(o + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
  }
}

}  // namespace

hipError_t launch_dequant(const DequantArgs& a, hipStream_t stream) {
  if (a.nrows <= 0) return hipSuccess;
  dim3 grid((unsigned)((a.nrows + kRowsPerTile - 1) / kRowsPerTile), a.batch * a.kv_heads * 2);
  hipLaunchKernelGGL(dequant_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace semkv
