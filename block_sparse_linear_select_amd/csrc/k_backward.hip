// Launcher of the backward pass (bf16 inputs; the float32 instantiations live
// in k_backward_f32.hip).
#include "backward.hpp"

namespace hsa {

hipError_t launch_backward(const Shape& s, const void* q, const void* k, const void* v, const void* dout,
                           const void* uq, const void* uk, const void* wo, const int32_t* row_ptr,
                           const int32_t* col_idx, const Scratch& w, float* dq, float* dk, float* dv, int part,
                           hipStream_t st) {
  BwdArgs a{};
  a.N = s.N; a.N_pad = s.N_pad; a.T = s.T; a.H = s.H;
  a.nchunk = stream_chunks(s);
  a.tpc = (s.T + a.nchunk - 1) / a.nchunk;
  {  // key-side linear pass: blocks of 8 waves over chunks of key tiles, about one block per CU in all
    const int bhs = s.B * s.H;
    int nk = 256 / bhs;
    nk = nk < 1 ? 1 : nk;
    const int maxk = (s.T + 3) / 4;  // at least four tiles (one per wave pair) per block
    nk = nk > maxk ? maxk : nk;
    a.tpc_k = (s.T + nk - 1) / nk;
  }
  a.gt = s.gt; a.gh = s.gh; a.gw = s.gw;
  a.scale = s.scale;
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.uq = uq; a.uk = uk; a.wo = wo;
  a.row_ptr = row_ptr; a.col_idx = col_idx;
  a.os = w.os; a.lse = w.lse; a.dsum = w.dsum; a.z = w.z; a.s_frag = w.s_full; a.s_pfrag = w.s_pfrag;
  a.wob_frag = w.wob_frag; a.uqp_frag = w.uqp_frag; a.ukp_frag = w.ukp_frag;
  a.uq_frag = w.uq_frag; a.uk_frag = w.uk_frag; a.rope = w.rope;
  a.part_ds = w.part_ds; a.part_dz = w.part_dz; a.ds_plain = w.ds_plain; a.ds_frag = w.ds_frag; a.dz = w.dz;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.nrows = (long)s.B * s.H * s.T;
  if (s.dt == Dt::F32)
    return launch_bwd_f32(s, a, w.csc_cnt, w.col_ptr, w.row_idx, w.csc_bits, w.csc_cap, part == 1, st);
  if (part == 1) return bwd_linear_by_shape<bf16_t>(s, a, st);
  return bwd_sparse<bf16_t>(s, a, w.csc_cnt, w.col_ptr, w.row_idx, w.csc_bits, w.csc_cap, st);
}

}  // namespace hsa
