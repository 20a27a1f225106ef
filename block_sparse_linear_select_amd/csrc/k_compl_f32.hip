// float32 instantiations of the complement-key linear branch (the tiny
// float32 workload).
#include "compl.hpp"

namespace hsa {

hipError_t launch_compl_f32(const Shape& s, const ComplArgs& a, hipStream_t st) {
  return compl_by_shape<float, float>(s, a, st);
}

}  // namespace hsa
