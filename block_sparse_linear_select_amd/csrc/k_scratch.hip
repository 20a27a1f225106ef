// Static device scratch of the allocation-free hybrid call
// (hsa_hybrid_attn_noalloc): a file-scope device array that the library
// never allocates at run time.  Its device address differs per GPU, so it is
// taken once per device with hipGetSymbolAddress (with that device current)
// and kept; host code uses only that address, never the array's name.
#include <mutex>
#include <vector>

#include "kernels.hpp"

namespace hsa {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

hipError_t static_scratch(void** out) {
  static std::mutex mu;
  static std::vector<void*> ptr;  // per device, taken on the first call there
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  if ((int)ptr.size() <= dev) ptr.resize((size_t)dev + 1, nullptr);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

}  // namespace hsa
