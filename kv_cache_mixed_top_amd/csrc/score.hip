// Key-norm token scores (SemKV Fig. 2: a per-token importance score from one
// model-internal indicator, ranked within the prompt; SemKV Table 3 lists the
// key-norm indicator).  score[b][t] = sum over a window of layers and every
// KV head of the Euclidean norm of token t's key row, accumulated in fp32
// layer by layer, head by head (the same order for every token).
//
// Workgroup = 256 threads = 64 tokens x 4 lanes.  Lane q of a token reads the
// 16-byte pieces at byte offsets 16q + 64i (i = 0..3) of each of the token's
// rows, so one load instruction of a quad covers 64 contiguous bytes and the
// 64 rows of one (layer, head) are one 16 KB run when the tokens are
// contiguous.  The (layer, head) rows are streamed kAhead at a time: all
// their loads are issued before the first is used.  Squares are summed by
// mixed-precision fmas straight from fp16 (the products are exact in fp32).
#include "semkv_internal.h"

namespace semkv {
namespace {

constexpr int kTok = 64;
constexpr int kThreads = 256;
constexpr int kAhead = 4;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  return x;   // the same value on the quad's four lanes
}

__global__ __launch_bounds__(kThreads) void score_keynorm_kernel(ScoreArgs a) {
  const int tid = threadIdx.x;
  const int r = tid >> 2, q = tid & 3;
  const int b = blockIdx.y;
  const int64_t t = (int64_t)blockIdx.x * kTok + r;
  const bool valid = t < a.n;
  const int total = a.nlayers * a.kv_heads;
  const uint16_t* base = a.k + (int64_t)b * a.sb + t * a.st + 8 * q;

  float acc = 0.0f;
  for (int j0 = 0; j0 < total; j0 += kAhead) {
    uint4 w[kAhead][4];
#pragma unroll
    for (int j = 0; j < kAhead; ++j) {
      const int lh = j0 + j;
      if (valid && lh < total) {
        const int layer = a.layer0 + lh / a.kv_heads;
        const int head = lh % a.kv_heads;
        const uint16_t* src = base + (int64_t)layer * a.sl + (int64_t)head * a.sh;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[j][i] = *reinterpret_cast<const uint4*>(src + 32 * i);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[j][i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int j = 0; j < kAhead; ++j) {
      float ss = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t ws[4] = {w[j][i].x, w[j][i].y, w[j][i].z, w[j][i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const half2_t h = __builtin_bit_cast(half2_t, ws[e]);
          ss = fmaf((float)h[0], (float)h[0], ss);
          ss = fmaf((float)h[1], (float)h[1], ss);
        }
      }
      ss = quad_sum(ss);
      if (j0 + j < total) acc += __builtin_sqrtf(ss);
    }
  }
  if (valid && q == 0) a.scores[(int64_t)b * a.ld + t] = acc;
}

// ---- hidden-state delta norm (SemKV Table 2's default indicator; Fig. 10:
// O(1) per token).  score[b][t] = sum_{j=1..S} ||h_j[t] - h_{j-1}[t]||_2 over
// the hidden states h_0 .. h_S of token t entering and leaving the last S
// layers.  One wave per token; lane l covers dimensions 8 l + 512 c of
// chunk c, reading the S + 1 states' 16 bytes of a chunk together (two
// chunks of loads in flight).  Each update is formed in fp32 from the two
// fp16 values (one rounding) and squared into a per-layer fp32 sum; the
// sums are reduced across the wave, square-rooted and added in layer order.
template <int S>
__global__ __launch_bounds__(kThreads) void score_hidden_delta_kernel(DeltaArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (t >= a.n) return;                                   // whole waves
  const uint16_t* base = a.h + (int64_t)b * a.sb + t * a.st + 8 * lane;
  float acc[S];
#pragma unroll
  for (int j = 0; j < S; ++j) acc[j] = 0.0f;
  auto load = [&](int c, uint4 (&x)[S + 1]) {
    const int off = 512 * c;
    const bool in = off + 8 * lane < a.d;
#pragma unroll
    for (int j = 0; j <= S; ++j)
      x[j] = in ? *reinterpret_cast<const uint4*>(base + (int64_t)j * a.ss + off) : make_uint4(0u, 0u, 0u, 0u);
  };
  auto accumulate = [&](const uint4 (&x)[S + 1]) {
#pragma unroll
    for (int j = 1; j <= S; ++j) {
      const uint32_t hi[4] = {x[j].x, x[j].y, x[j].z, x[j].w};
      const uint32_t lo[4] = {x[j - 1].x, x[j - 1].y, x[j - 1].z, x[j - 1].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const half2_t u = __builtin_bit_cast(half2_t, hi[e]), v = __builtin_bit_cast(half2_t, lo[e]);
        const float d0 = (float)u[0] - (float)v[0], d1 = (float)u[1] - (float)v[1];
        acc[j - 1] = fmaf(d0, d0, acc[j - 1]);
        acc[j - 1] = fmaf(d1, d1, acc[j - 1]);
      }
    }
  };
  const int chunks = (a.d + 511) / 512;
  int c = 0;
  for (; c + 2 <= chunks; c += 2) {
    uint4 x0[S + 1], x1[S + 1];
    load(c, x0);
    load(c + 1, x1);
    accumulate(x0);
    accumulate(x1);
  }
  if (c < chunks) {
    uint4 x0[S + 1];
    load(c, x0);
    accumulate(x0);
  }
  float score = 0.0f;
#pragma unroll
  for (int j = 0; j < S; ++j) {
    float v = acc[j];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    score += __builtin_sqrtf(v);
  }
  if (lane == 0) a.scores[(int64_t)b * a.ld + t] = score;
}

}  // namespace

hipError_t launch_score_hidden_delta(const DeltaArgs& a, int batch, hipStream_t stream) {
  const dim3 grid((unsigned)((a.n + kThreads / 64 - 1) / (kThreads / 64)), (unsigned)batch);
  switch (a.S) {
#define SEMKV_DELTA(K)                                                                          \
  case K:                                                                                       \
    hipLaunchKernelGGL(score_hidden_delta_kernel<K>, grid, dim3(kThreads), 0, stream, a);     \
    break;
    SEMKV_DELTA(1) SEMKV_DELTA(2) SEMKV_DELTA(3) SEMKV_DELTA(4)
    SEMKV_DELTA(5) SEMKV_DELTA(6) SEMKV_DELTA(7) SEMKV_DELTA(8)
#undef SEMKV_DELTA
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_score_keynorm(const ScoreArgs& a, int batch, hipStream_t stream) {
  const dim3 grid((unsigned)((a.n + kTok - 1) / kTok), (unsigned)batch);
  hipLaunchKernelGGL(score_keynorm_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace semkv
