// Launcher of the complement-key linear branch (bf16 and fp8 inputs; the
// float32 instantiations live in k_compl_f32.hip).
#include "compl.hpp"

namespace hsa {

hipError_t launch_compl(const Shape& s, const void* q, const float* qs, const int32_t* row_ptr,
                        const int32_t* col_idx, const Scratch& w, void* o, bool add, hipStream_t st) {
  ComplArgs a{};
  a.N = s.N; a.N_pad = s.N_pad; a.T = s.T; a.H = s.H;
  a.gt = s.gt; a.gh = s.gh; a.gw = s.gw;
  a.q = q; a.qs = qs; a.row_ptr = row_ptr; a.col_idx = col_idx;
  a.tile_s = w.tile_s; a.tile_z = w.tile_z; a.s_full = w.s_full; a.z = w.z;
  a.uq_frag = w.uq_frag; a.wo_frag = w.wo_frag; a.rope = w.rope;
  a.o = o;
  a.add = add ? 1 : 0;
  a.nrows = (long)s.B * s.H * s.T;
  switch (s.dt) {
    case Dt::F32: return launch_compl_f32(s, a, st);
    case Dt::BF16: return compl_by_shape<bf16_t, bf16_t>(s, a, st);
    default: return compl_by_shape<fp8_t, bf16_t>(s, a, st);
  }
}

}  // namespace hsa
