// Launcher of the query-tile kernel (bf16 inputs; the float32 instantiations
// live in k_attend_f32.hip).
#include "attend.hpp"

namespace hsa {

// ------------------------------------------------------------- launcher
hipError_t launch_attend(const Shape& s, const void* q, const void* k, const void* v,
                         const float* qs, const float* ks, const float* vs,
                         const int32_t* row_ptr, const int32_t* col_idx, bool sparse, bool linear,
                         const Scratch& w, void* o, float* lse, hipStream_t st, void* o_s) {
  AttendArgs a{};
  a.N = s.N; a.N_pad = s.N_pad; a.T = s.T; a.H = s.H;
  a.gt = s.gt; a.gh = s.gh; a.gw = s.gw;
  a.scale_log2 = s.scale * kLog2e;
  a.q = q; a.k = k; a.v = v; a.row_ptr = row_ptr; a.col_idx = col_idx;
  a.sp_frag = w.sp_frag; a.z = w.z; a.uq_frag = w.uq_frag; a.rope = w.rope; a.vt = w.vt;
  a.qs = qs; a.ks = ks; a.vs = vs;
  a.o = o; a.lse = lse; a.o_s = o_s;
  a.nrows = (long)s.B * s.H * s.T;
  switch (s.dt) {
    case Dt::F32: return launch_attend_f32(s, a, sparse, linear, st);
    case Dt::BF16: return attend_bf16_by_shape(s, a, sparse, linear, st);
    default: return attend_fp8_by_shape(s, a, sparse, linear, st);
  }
}

}  // namespace hsa
