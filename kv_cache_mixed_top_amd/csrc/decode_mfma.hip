// Launchers of the matrix-core decode (kernels in decode_mfma_kernel.h):
// level-pair dispatch, occupancy, and the shapes the kernels accept.
#include <atomic>

#include "decode_mfma_kernel.h"

namespace semkv {
namespace {

// Level pairs (high, low) with a matrix-core kernel; a pool with no rows
// takes the other pool's level count.  Pairs with 16 levels and the rest of
// the 3- and 8-level pairs are instantiated in decode_mfma_wide.hip.
template <bool kRot>
hipError_t launch_pair(int LA, int LB, dim3 grid, const DecodeArgs& a, hipStream_t stream) {
#define SEMKV_PAIR(X, Y) \
  if (LA == X && LB == Y) return launch_mfma<X, Y, kRot>(grid, a, stream);
  SEMKV_PAIR(6, 5) SEMKV_PAIR(6, 6) SEMKV_PAIR(5, 5) SEMKV_PAIR(5, 4) SEMKV_PAIR(4, 4)
  SEMKV_PAIR(6, 4) SEMKV_PAIR(4, 3) SEMKV_PAIR(3, 3) SEMKV_PAIR(8, 8) SEMKV_PAIR(8, 6)
#undef SEMKV_PAIR
  return launch_decode_mfma_wide(LA, LB, kRot, grid, a, stream);
}

bool fast_level(int L) { return L == 3 || L == 4 || L == 5 || L == 6 || L == 8 || L == 16; }

void effective_pair(const DecodeArgs& a, int& LA, int& LB) {
  LA = a.fmt[0].L;
  LB = a.fmt[1].L;
  if (a.rows[0] == 0) LA = LB;
  if (a.rows[1] == 0) LB = LA;
}

}  // namespace

// Workgroups of the matrix-core kernel resident on the current device at
// once (registers and LDS both limit it; the 6/5-level kernel stands for
// all); the pool chunking fills them once.  Cached per device ordinal;
// concurrent first calls compute the same value.
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
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_mfma_kernel<6, 5, false>, 128, 0) !=
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
  int LA, LB;
  effective_pair(a, LA, LB);
  if (!fast_level(LA) || !fast_level(LB) || LA < LB) return false;
  // the PV sums of a chunk stay exact in int32 (< 2^21 per tile and column)
  if (a.chunk > 16384) return false;
  for (int s = 0; s < 2; ++s)
    if (a.cap[s] * 64 >= ((int64_t)1 << 31)) return false;   // 32-bit row offsets in the kernels
  return true;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, bool with_tail, hipStream_t stream) {
  const int chunks = a.nch[0] + a.nch[1] + (with_tail ? a.nch[2] : 0);
  if (chunks == 0) return hipSuccess;
  int LA, LB;
  effective_pair(a, LA, LB);
  dim3 grid(chunks, a.nl * a.kv_heads, a.batch);
  return a.rotate ? launch_pair<true>(LA, LB, grid, a, stream) : launch_pair<false>(LA, LB, grid, a, stream);
}

}  // namespace semkv
