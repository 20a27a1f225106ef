// Launchers of the streaming pass and the state finalize (bf16 and fp8
// inputs; the float32 instantiations live in k_stream_f32.hip).
#include "stream.hpp"

namespace hsa {

// ------------------------------------------------------------- launchers
hipError_t launch_rope_table(const Shape& s, float2* tab, hipStream_t st) {
  int n = rope_entries(s);
  k_rope_table<<<(n + 255) / 256, 256, 0, st>>>(s.gt, s.gh, s.gw, s.rank, (double)s.rope_base, tab);
  return hipGetLastError();
}

hipError_t launch_stream_pass(const Shape& s, const void* q, const void* k, const void* v,
                              const float* qs, const float* ks, const float* vs,
                              const void* uk, bool pool, bool state, const Scratch& w,
                              double* kbar_out, hipStream_t st) {
  StreamArgs a{};
  a.N = s.N; a.N_pad = s.N_pad; a.T = s.T;
  a.nchunk = stream_chunks(s);
  a.tpc = (s.T + a.nchunk - 1) / a.nchunk;
  a.gt = s.gt; a.gh = s.gh; a.gw = s.gw;
  a.q = q; a.k = k; a.v = v; a.qs = qs; a.ks = ks; a.vs = vs; a.uk = uk; a.H = s.H;
  a.kmean = w.kmean; a.khi = w.khi; a.klo = w.klo; a.kbar_out = kbar_out;
  a.part_s = w.part_s; a.part_z = w.part_z; a.rope = w.rope; a.vt = w.vt;
  if (state && s.compl_keys) { a.tile_s = w.tile_s; a.tile_z = w.tile_z; }
  a.nrope = rope_entries(s);
  switch (s.dt) {
    case Dt::F32: return launch_stream_f32(s, a, pool, state, st);
    case Dt::BF16: return stream_by_shape<bf16_t, bf16_t>(s, a, pool, state, st);
    default: return stream_by_shape<fp8_t, bf16_t>(s, a, pool, state, st);
  }
}

hipError_t launch_finalize(const Shape& s, const void* uq, const void* wo, const Scratch& w, hipStream_t st) {
  FinalArgs a{};
  a.nchunk = stream_chunks(s); a.H = s.H; a.B = s.B;
  a.part_s = w.part_s; a.part_z = w.part_z; a.wo = wo; a.uq = uq;
  a.sp_frag = w.sp_frag; a.z = w.z; a.uq_frag = w.uq_frag;
  if (s.compl_keys) { a.s_full = w.s_full; a.wo_frag = w.wo_frag; }
  if (w.s_pfrag) {  // backward pass
    a.s_full = w.s_full; a.s_pfrag = w.s_pfrag; a.wob_frag = w.wob_frag; a.uqp_frag = w.uqp_frag;
  }
  if (s.dt == Dt::F32) return launch_finalize_f32(s, a, st);
  return finalize_by_shape<bf16_t>(s, a, st);
}

hipError_t launch_vtranspose(const Shape& s, const void* v, const Scratch& w, hipStream_t st) {
  dim3 grid(s.T, s.B * s.H);
  k_vtranspose_fp8<<<grid, 256, 0, st>>>(s.N, s.N_pad, s.T, reinterpret_cast<const fp8_t*>(v),
                                          reinterpret_cast<uint8_t*>(w.vt));
  return hipGetLastError();
}

// ------------------------------------------------------- read calibration
// A plain streaming read of a device buffer: 16-byte loads, eight per thread
// in flight, grid-stride, folded into one word per thread.  It reaches the
// read rate a simple kernel gets from this GPU's memory, the practical
// ceiling against which the streaming pass (one read of K and V) is measured.
static __global__ __launch_bounds__(256) void k_read_calibrate(const u32x4* __restrict__ p, size_t n,
                                                                uint32_t* __restrict__ sink) {
  constexpr int U = 8;
  size_t i = (size_t)blockIdx.x * 256 * U + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256 * U;
  uint32_t acc = 0;
  for (; i + (U - 1) * 256 < n; i += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * 256);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  // the group that does not fit whole (every later group starts past n)
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (i + u * 256 < n) {
      const u32x4 t = p[i + u * 256];
      acc ^= t[0] ^ t[1] ^ t[2] ^ t[3];
    }
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

hipError_t launch_read_calibrate(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st) {
  k_read_calibrate<<<kReadCalibrateBlocks, 256, 0, st>>>(reinterpret_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace hsa
