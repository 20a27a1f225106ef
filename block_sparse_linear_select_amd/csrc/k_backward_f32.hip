// float32 instantiations of the backward pass (the tiny float32 workload).
#include "backward.hpp"

namespace hsa {

hipError_t launch_bwd_f32(const Shape& s, const BwdArgs& a, int32_t* csc_cnt, int32_t* col_ptr, int32_t* row_idx,
                          uint32_t* bits, long cap, bool linear_part, hipStream_t st) {
  if (linear_part) return bwd_linear_by_shape<float>(s, a, st);
  return bwd_sparse<float>(s, a, csc_cnt, col_ptr, row_idx, bits, cap, st);
}

}  // namespace hsa
