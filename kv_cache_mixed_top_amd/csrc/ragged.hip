// Per-sequence counters of a ragged batch (SemKV page, Fig. 6: each prompt is
// ranked and quantized on its own, each sequence's generation blocks fill and
// are quantized independently; Table 2: multi-turn use flushes at each turn's
// end).  Sequence b's counters are kSeqWords int64 in device memory:
// n_high, n_low, n_tail, n_tokens, status.  These small kernels advance them
// in stream order after the kernels that read them as offsets, so that a
// whole ragged step runs without the host knowing any sequence's length.
#include "semkv_internal.h"

namespace semkv {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void seq_reset_kernel(int64_t* seq, int batch) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < batch * kSeqWords) seq[i] = 0;
}

// The same decisions as pool_part in quantize.hip: a prompt is written only
// while the sequence's tail is empty and if both pools have room.
__global__ __launch_bounds__(kThreads) void seq_prefill_advance_kernel(int64_t* seq, const int32_t* n_seq,
                                                                       double r, int batch, int64_t cap_high,
                                                                       int64_t cap_low) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= batch) return;
  int64_t* sq = seq + (int64_t)b * kSeqWords;
  const int64_t n = n_seq[b];
  if (n <= 0) return;
  const int64_t k = topr_count(n, r);
  if (sq[kSeqTail] != 0) {
    sq[kSeqStatus] |= kSeqTailBusy;
  } else if (sq[kSeqHigh] + k > cap_high || sq[kSeqLow] + (n - k) > cap_low) {
    sq[kSeqStatus] |= kSeqCapacity;
  } else {
    sq[kSeqHigh] += k;
    sq[kSeqLow] += n - k;
    sq[kSeqTokens] += n;
  }
}

// After the append kernel (which wrote at n_tail when active and n_tail <
// block): count the token, then decide whether the tail is quantized now.
__global__ __launch_bounds__(kThreads) void seq_tail_plan_kernel(int64_t* seq, const int32_t* active,
                                                                 const int32_t* flush, double r, int block,
                                                                 int batch, int64_t cap_high,
                                                                 int64_t cap_low, int32_t* nq) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= batch) return;
  int64_t* sq = seq + (int64_t)b * kSeqWords;
  int64_t nt = sq[kSeqTail];
  if (active && active[b] != 0) {
    if (nt < block) {
      nt += 1;
      sq[kSeqTokens] += 1;
    } else {
      sq[kSeqStatus] |= kSeqTailFull;   // the token was dropped
    }
  }
  sq[kSeqTail] = nt;
  int64_t n = (nt == block || (flush && flush[b] != 0 && nt > 0)) ? nt : 0;
  if (n > 0) {
    const int64_t k = topr_count(n, r);
    if (sq[kSeqHigh] + k > cap_high || sq[kSeqLow] + (n - k) > cap_low) {
      sq[kSeqStatus] |= kSeqCapacity;
      n = 0;
    }
  }
  nq[b] = (int32_t)n;
}

__global__ __launch_bounds__(kThreads) void seq_tail_advance_kernel(int64_t* seq, const int32_t* nq,
                                                                    double r, int batch) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= batch) return;
  const int64_t n = nq[b];
  if (n <= 0) return;
  int64_t* sq = seq + (int64_t)b * kSeqWords;
  const int64_t k = topr_count(n, r);
  sq[kSeqHigh] += k;
  sq[kSeqLow] += n - k;
  sq[kSeqTail] = 0;
}

dim3 seq_grid(int batch) { return dim3((unsigned)((batch * kSeqWords + kThreads - 1) / kThreads)); }

}  // namespace

hipError_t launch_seq_reset(int64_t* seq, int batch, hipStream_t stream) {
  hipLaunchKernelGGL(seq_reset_kernel, seq_grid(batch), dim3(kThreads), 0, stream, seq, batch);
  return hipGetLastError();
}

hipError_t launch_seq_prefill_advance(int64_t* seq, const int32_t* n_seq, double r, int batch,
                                      int64_t cap_high, int64_t cap_low, hipStream_t stream) {
  hipLaunchKernelGGL(seq_prefill_advance_kernel, seq_grid(batch), dim3(kThreads), 0, stream, seq, n_seq, r,
                     batch, cap_high, cap_low);
  return hipGetLastError();
}

hipError_t launch_seq_tail_plan(int64_t* seq, const int32_t* active, const int32_t* flush,
                                double r, int block, int batch, int64_t cap_high, int64_t cap_low,
                                int32_t* nq, hipStream_t stream) {
  hipLaunchKernelGGL(seq_tail_plan_kernel, seq_grid(batch), dim3(kThreads), 0, stream, seq, active, flush, r,
                     block, batch, cap_high, cap_low, nq);
  return hipGetLastError();
}

hipError_t launch_seq_tail_advance(int64_t* seq, const int32_t* nq, double r, int batch,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(seq_tail_advance_kernel, seq_grid(batch), dim3(kThreads), 0, stream, seq, nq, r, batch);
  return hipGetLastError();
}

}  // namespace semkv
