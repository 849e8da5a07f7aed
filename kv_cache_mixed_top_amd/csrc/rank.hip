// Top-r ranking of per-token importance scores (SemKV page, Fig. 2: ranking
// within each prompt without score normalisation; Fig. 4: the top-r tokens
// form the high-precision set H, no threshold is estimated).
//
// Order: score descending, equal scores by lower token index, -0 == +0, NaN
// below every number.  Scores map to a monotone uint32 key; the k-th largest
// key T is found by an 8-bit radix select; H = {key > T} plus the first
// (k - #{key > T}) tokens with key == T in index order.  perm lists H in
// ascending order, then the rest ascending.
//
// Three kernels:
//  * rank_select32_kernel -- one 1024-thread workgroup per sequence for
//                            n <= 32,768: each thread keeps the keys of its
//                            32 tokens in registers for every pass
//  * rank_select_kernel   -- one 1024-thread workgroup per sequence, any n
//  * rank_block_kernel    -- one wave64 per sequence for n <= 128 (generation
//                            blocks): bitonic sort of 64-bit (key, ~index)
//                            composites held two per lane.
#include "semkv_internal.h"

namespace semkv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// Ragged batches: sequence b ranks its first n_seq[b] (at most n) scores
// with its own k = floor(r n_seq[b] + 1/2); perm rows have stride ld_perm
// and mask rows (n + 31) / 32 words, n being the bound of the launch.
struct RaggedRank {
  const int32_t* n_seq;
  double r;
  int64_t ld_perm;
  __device__ void apply(int b, int& n, int& k) const {
    n = min(n_seq[b], n);
    k = (int)topr_count(n, r);
  }
};

__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 0u;                 // NaN: below every number
  if ((u << 1) == 0u) u = 0u;            // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of one value per thread over the workgroup.
__device__ int block_exclusive_scan(int v, int* buf, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) buf[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kWaves ? buf[lane] : 0;
    int wi = w;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int t = __shfl_up(wi, o, 64);
      if (lane >= o) wi += t;
    }
    if (lane < kWaves) buf[lane] = wi - w;
    if (lane == kWaves - 1) buf[kWaves] = wi;
  }
  __syncthreads();
  const int res = buf[wave] + incl - v;
  *total = buf[kWaves];
  __syncthreads();
  return res;
}

__global__ __launch_bounds__(kThreads) void rank_select_kernel(
    const float* __restrict__ scores, int64_t ld, int n, int k, int items,
    int32_t* __restrict__ perm, uint32_t* __restrict__ mask, RaggedRank rg) {
  __shared__ uint32_t hist[kWaves][256];
  __shared__ int scan_buf[kWaves + 1];
  __shared__ uint32_t sh_prefix;
  __shared__ int sh_remaining;

  const int b = blockIdx.x;
  const float* s = scores + (int64_t)b * ld;
  int32_t* p = perm + (int64_t)b * (rg.ld_perm > 0 ? rg.ld_perm : n);
  uint32_t* mk = mask ? mask + (int64_t)b * ((n + 31) >> 5) : nullptr;
  if (rg.n_seq) rg.apply(b, n, k);
  if (n <= 0) return;
  const int tid = threadIdx.x, wave = tid >> 6;

  // -- radix select of the k-th largest key (k >= 1)
  uint32_t thr = 0xFFFFFFFFu;
  int need_eq = 0;
  if (k > 0) {
    uint32_t prefix = 0, pmask = 0;
    int remaining = k;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < kWaves * 256; i += kThreads) (&hist[0][0])[i] = 0u;
      __syncthreads();
      for (int i = tid; i < n; i += kThreads) {          // order-free: coalesced
        const uint32_t key = score_key(s[i]);
        if ((key & pmask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 256) {
        uint32_t t = 0;
        for (int w = 0; w < kWaves; ++w) t += hist[w][tid];
        hist[0][tid] = t;
      }
      __syncthreads();
      if (tid == 0) {
        int cum = 0, d = 255;
        for (; d > 0; --d) {
          const int c = (int)hist[0][d];
          if (cum + c >= remaining) break;
          cum += c;
        }
        sh_prefix = prefix | ((uint32_t)d << shift);
        sh_remaining = remaining - cum;
      }
      __syncthreads();
      prefix = sh_prefix;
      remaining = sh_remaining;
      pmask |= 0xFFu << shift;
      __syncthreads();
    }
    thr = prefix;
    need_eq = remaining;
  }

  // -- membership and stable partition, each thread owns [begin, end)
  const int begin = tid * items;
  const int end = min(begin + items, n);
  int gt = 0, eq = 0;
  if (k > 0) {
    for (int i = begin; i < end; ++i) {
      const uint32_t key = score_key(s[i]);
      gt += key > thr;
      eq += key == thr;
    }
  }
  int eq_total;
  const int eq_before = block_exclusive_scan(eq, scan_buf, &eq_total);
  const int take_eq = min(max(need_eq - eq_before, 0), eq);
  int in_total;
  const int in_before = block_exclusive_scan(gt + take_eq, scan_buf, &in_total);

  int pin = in_before;
  int pout = k + (begin - in_before);
  int eq_seen = 0;
  uint32_t word = 0;
  for (int i = begin; i < end; ++i) {
    bool in = false;
    if (k > 0) {
      const uint32_t key = score_key(s[i]);
      if (key > thr) {
        in = true;
      } else if (key == thr) {
        in = (eq_before + eq_seen) < need_eq;
        ++eq_seen;
      }
    }
    if (in) {
      if (pin < k) p[pin] = i;
      ++pin;
    } else {
      if (pout < n) p[pout] = i;
      ++pout;
    }
    word |= (uint32_t)in << (i & 31);
    if ((i & 31) == 31 || i == end - 1) {
      if (mk) mk[i >> 5] = word;
      word = 0;
    }
  }
}

// The same selection and partition for n <= 32 * kThreads, with the keys of
// tokens [32 tid, 32 tid + 32) loaded once (independent loads, one memory
// latency) and the radix digit found by a parallel scan of the 256 bins.
__global__ __launch_bounds__(kThreads) void rank_select32_kernel(
    const float* __restrict__ scores, int64_t ld, int n, int k, int32_t* __restrict__ perm,
    uint32_t* __restrict__ mask, RaggedRank rg) {
  constexpr int kItems = 32;
  __shared__ uint32_t hist[kWaves][256];
  __shared__ int scan_buf[kWaves + 1];
  __shared__ uint32_t sh_prefix;
  __shared__ int sh_remaining;

  const int b = blockIdx.x;
  const float* s = scores + (int64_t)b * ld;
  int32_t* p = perm + (int64_t)b * (rg.ld_perm > 0 ? rg.ld_perm : n);
  uint32_t* mk = mask ? mask + (int64_t)b * ((n + 31) >> 5) : nullptr;
  if (rg.n_seq) rg.apply(b, n, k);
  if (n <= 0) return;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int begin = tid * kItems;
  const int cnt = max(0, min(kItems, n - begin));
  uint32_t key[kItems];
  if (cnt == kItems && ((uintptr_t)(s + begin) & 15u) == 0) {   // 16-byte loads
#pragma unroll
    for (int j = 0; j < kItems / 4; ++j) {
      const float4 v = reinterpret_cast<const float4*>(s + begin)[j];
      key[4 * j] = score_key(v.x);
      key[4 * j + 1] = score_key(v.y);
      key[4 * j + 2] = score_key(v.z);
      key[4 * j + 3] = score_key(v.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kItems; ++j) key[j] = j < cnt ? score_key(s[begin + j]) : 0u;
  }

  // -- radix select of the k-th largest key (k >= 1)
  uint32_t thr = 0xFFFFFFFFu;
  int need_eq = 0;
  if (k > 0) {
    uint32_t prefix = 0, pmask = 0;
    int remaining = k;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < kWaves * 256; i += kThreads) (&hist[0][0])[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kItems; ++j)
        if (j < cnt && (key[j] & pmask) == prefix)
          atomicAdd(&hist[wave][(key[j] >> shift) & 255u], 1u);
      __syncthreads();
      // thread t < 256 takes digit 255 - t; the exclusive scan gives the
      // candidates above it, and the digit where the count reaches
      // `remaining` is the next digit of the k-th largest key
      int c = 0;
      if (tid < 256) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) c += (int)hist[w][255 - tid];
      }
      int total;
      const int above = block_exclusive_scan(c, scan_buf, &total);
      if (tid < 256 && above < remaining && remaining <= above + c) {
        sh_prefix = prefix | ((uint32_t)(255 - tid) << shift);
        sh_remaining = remaining - above;
      }
      __syncthreads();
      prefix = sh_prefix;
      remaining = sh_remaining;
      pmask |= 0xFFu << shift;
      __syncthreads();
    }
    thr = prefix;
    need_eq = remaining;
  }

  // -- membership and stable partition of the thread's tokens
  int gt = 0, eq = 0;
  if (k > 0) {
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      gt += j < cnt && key[j] > thr;
      eq += j < cnt && key[j] == thr;
    }
  }
  int eq_total;
  const int eq_before = block_exclusive_scan(eq, scan_buf, &eq_total);
  const int take_eq = min(max(need_eq - eq_before, 0), eq);
  int in_total;
  const int in_before = block_exclusive_scan(gt + take_eq, scan_buf, &in_total);

  int pin = in_before;
  int pout = k + (begin - in_before);
  int eq_seen = 0;
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    if (j < cnt) {
      bool in = false;
      if (k > 0) {
        if (key[j] > thr) {
          in = true;
        } else if (key[j] == thr) {
          in = (eq_before + eq_seen) < need_eq;
          ++eq_seen;
        }
      }
      if (in) {
        if (pin < k) p[pin] = begin + j;
        ++pin;
      } else {
        if (pout < n) p[pout] = begin + j;
        ++pout;
      }
      word |= (uint32_t)in << j;
    }
  }
  if (mk && cnt > 0) mk[tid] = word;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)v, src, 64);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), src, 64);
  return ((uint64_t)hi << 32) | lo;
}

// One wave per sequence, n <= 128.  Element e = j*64 + lane (j = 0, 1).
__global__ __launch_bounds__(64) void rank_block_kernel(
    const float* __restrict__ scores, int64_t ld, int n, int k,
    int32_t* __restrict__ perm, uint32_t* __restrict__ mask, RaggedRank rg) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const float* s = scores + (int64_t)b * ld;
  int32_t* p = perm + (int64_t)b * (rg.ld_perm > 0 ? rg.ld_perm : n);
  const int mask_ld = (n + 31) >> 5;
  if (rg.n_seq) rg.apply(b, n, k);
  if (n <= 0) return;
  const int nwords = (n + 31) >> 5;

  // composite: higher is better; ties resolved by the lower index
  uint64_t orig[2], key[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = j * 64 + lane;
    uint64_t c = 0;   // padding ranks below every real token (NaN included)
    if (t < n) c = ((uint64_t)score_key(s[t]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)t);
    orig[j] = key[j] = c;
  }
  // bitonic sort, descending
  for (int size = 2; size <= 128; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      uint64_t nk[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int e = j * 64 + lane;
        const uint64_t other = (stride == 64) ? key[j ^ 1] : shfl_xor_u64(key[j], stride);
        const bool lower = (e & stride) == 0;
        const bool desc = (e & size) == 0;
        const bool keep_max = (lower == desc);
        const uint64_t mine = key[j];
        nk[j] = keep_max ? (mine > other ? mine : other) : (mine < other ? mine : other);
      }
      key[0] = nk[0];
      key[1] = nk[1];
    }
  }
  uint64_t thr = ~0ull;
  if (k > 0) {
    const int pos = k - 1;
    thr = shfl_u64((pos >> 6) ? key[1] : key[0], pos & 63);
  }
  const bool in0 = k > 0 && lane < n && orig[0] >= thr;
  const bool in1 = k > 0 && 64 + lane < n && orig[1] >= thr;
  const uint64_t b0 = __ballot(in0);
  const uint64_t b1 = __ballot(in1);
  if (mask) {
    uint32_t* mk = mask + (int64_t)b * mask_ld;
    const uint32_t w[4] = {(uint32_t)b0, (uint32_t)(b0 >> 32), (uint32_t)b1, (uint32_t)(b1 >> 32)};
    if (lane < nwords) mk[lane] = w[lane];
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  {
    const int t = lane;
    if (t < n) {
      const int before = __popcll(b0 & below);
      const int dst = in0 ? before : k + (t - before);
      if (dst >= 0 && dst < n) p[dst] = t;
    }
  }
  {
    const int t = 64 + lane;
    if (t < n) {
      const int before = __popcll(b0) + __popcll(b1 & below);
      const int dst = in1 ? before : k + (t - before);
      if (dst >= 0 && dst < n) p[dst] = t;
    }
  }
}

}  // namespace

hipError_t launch_rank(const float* scores, int batch, int n, int64_t ld, int k,
                       int32_t* perm, uint32_t* mask, hipStream_t stream, const int32_t* n_seq,
                       double r, int64_t ld_perm) {
  const RaggedRank rg{n_seq, r, ld_perm};
  if (n <= 128) {
    hipLaunchKernelGGL(rank_block_kernel, dim3(batch), dim3(64), 0, stream, scores, ld, n, k,
                       perm, mask, rg);
  } else if (n <= 32 * kThreads) {
    hipLaunchKernelGGL(rank_select32_kernel, dim3(batch), dim3(kThreads), 0, stream, scores, ld,
                       n, k, perm, mask, rg);
  } else {
    int items = (n + kThreads - 1) / kThreads;
    items = (items + 31) & ~31;   // each thread owns whole mask words
    hipLaunchKernelGGL(rank_select_kernel, dim3(batch), dim3(kThreads), 0, stream, scores, ld,
                       n, k, items, perm, mask, rg);
  }
  return hipGetLastError();
}

}  // namespace semkv
