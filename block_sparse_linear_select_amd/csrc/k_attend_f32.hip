// float32 instantiations of the query-tile kernel (the tiny float32
// workload).  Built at -O1: hipcc's -O3 backend crashes on them.
#include "attend.hpp"

namespace hsa {

hipError_t launch_attend_f32(const Shape& s, const AttendArgs& a, bool sparse, bool linear, hipStream_t st) {
  return attend_by_shape<float>(s, a, sparse, linear, st);
}

}  // namespace hsa
