// float32 instantiations of the streaming pass and the state finalize (the
// tiny float32 workload).  This translation unit is built at -O1: hipcc's
// -O3 backend crashes on the float32 pooling + state instantiation.
#include "stream.hpp"

namespace hsa {

hipError_t launch_stream_f32(const Shape& s, const StreamArgs& a, bool pool, bool state, hipStream_t st) {
  return stream_by_shape<float, float>(s, a, pool, state, st);
}

hipError_t launch_finalize_f32(const Shape& s, const FinalArgs& a, hipStream_t st) {
  return finalize_by_shape<float>(s, a, st);
}

}  // namespace hsa
