// Append newly generated tokens' fp16 K/V rows and scores to the tail
// (SemKV page, Fig. 6: the newest partial block stays fp16 while decoding and
// the scores of generated tokens accumulate until the block completes).
#include "semkv_internal.h"

namespace semkv {
namespace {

constexpr int kRowsPerBlock = 16;   // 16 lanes x 16 bytes per 256-byte row

__global__ __launch_bounds__(256) void append_tail_kernel(AppendArgs a) {
  const int64_t total = (int64_t)a.batch * a.layers * a.kv_heads * 2 * a.t_cnt;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);
  const int lane = threadIdx.x & 15;
  if (row < total) {
    int64_t rest = row;
    const int i = (int)(rest % a.t_cnt);
    rest /= a.t_cnt;
    const int kvsel = (int)(rest & 1);
    rest >>= 1;
    const int head = (int)(rest % a.kv_heads);
    rest /= a.kv_heads;
    const int layer = (int)(rest % a.layers);
    const int b = (int)(rest / a.layers);
    // ragged batch: only active sequences append, at their own tail length
    // (a full tail, left by a capacity failure, takes nothing more)
    int pos = a.pos;
    bool on = true;
    if (a.seq) {
      pos = (int)a.seq[(int64_t)b * kSeqWords + kSeqTail];
      on = a.active[b] != 0 && pos < a.block;
    }
    if (on) {
      const uint16_t* src = a.src[kvsel] + (int64_t)b * a.sb + (int64_t)layer * a.sl +
                            (int64_t)head * a.sh + (int64_t)(a.t_off + i) * a.st;
      uint16_t* dst = a.tail_kv +
                      (((((int64_t)b * a.layers + layer) * a.kv_heads + head) * 2 + kvsel) * a.block +
                       pos + i) * kHeadDim;
      reinterpret_cast<uint4*>(dst)[lane] = reinterpret_cast<const uint4*>(src)[lane];
    }
  }
  if (blockIdx.x == 0) {
    for (int j = threadIdx.x; j < a.batch * a.t_cnt; j += blockDim.x) {
      const int b = j / a.t_cnt, i = j - b * a.t_cnt;
      int pos = a.pos;
      if (a.seq) {
        pos = (int)a.seq[(int64_t)b * kSeqWords + kSeqTail];
        if (a.active[b] == 0 || pos >= a.block) continue;
      }
      a.tail_score[(int64_t)b * a.block + pos + i] = a.score_new[(int64_t)b * a.t_total + a.t_off + i];
    }
  }
}

}  // namespace

hipError_t launch_append_tail(const AppendArgs& a, hipStream_t stream) {
  const int64_t total = (int64_t)a.batch * a.layers * a.kv_heads * 2 * a.t_cnt;
  const int64_t blocks = (total + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(append_tail_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace semkv
