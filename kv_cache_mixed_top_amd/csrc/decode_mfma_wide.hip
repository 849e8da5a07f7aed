// Matrix-core decode: the level pairs with 16 levels, the 3-level pairs
// under 5 and 6 levels and the 8-level pairs other than (8,8) and (8,6) (the
// others are in decode_mfma.hip; the kernels are in
// decode_mfma_kernel.h).  A separate translation unit so that the pairs
// compile in parallel.
#include "decode_mfma_kernel.h"

namespace semkv {

hipError_t launch_decode_mfma_wide(int LA, int LB, bool rot, dim3 grid, const DecodeArgs& a,
                                   hipStream_t stream) {
#define SEMKV_PAIR(X, Y)                                                                     \
  if (LA == X && LB == Y)                                                                    \
    return rot ? launch_mfma<X, Y, true>(grid, a, stream) : launch_mfma<X, Y, false>(grid, a, stream);
  SEMKV_PAIR(16, 16) SEMKV_PAIR(16, 6) SEMKV_PAIR(16, 5) SEMKV_PAIR(16, 4) SEMKV_PAIR(16, 3)
  SEMKV_PAIR(6, 3) SEMKV_PAIR(5, 3) SEMKV_PAIR(16, 8) SEMKV_PAIR(8, 5) SEMKV_PAIR(8, 4)
  SEMKV_PAIR(8, 3)
#undef SEMKV_PAIR
  return hipErrorInvalidValue;
}

}  // namespace semkv
