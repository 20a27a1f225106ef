// Readout of the rotary low-rank linear branch for the queries of one wave
// (SparkDiffusion news article, section 05: the low-rank linear branch with
// rotary position information), shared by the query-tile kernels and the
// complement-key kernel, plus the fp8 code -> bf16 operand conversion.
#pragma once

#include "common.hpp"

namespace hsa {

// Operands of the readout of one (b, h).
template <typename T>
struct ReadoutSrc {
  const T* uq;        // U_q^T as A fragments of the head
  const T* sp;        // state (times W_o, or not) as A fragments: NFE values (float) or hi + lo halves (bf16)
  const float* z;     // [r] feature sum of the keys
  const float2* rope; // RoPE table
  int gt, gh, gw;     // latent grid
};

// 8 fp8 codes (two dwords) -> bf16 fragment with the exact code values
__device__ __forceinline__ void codes_to_bf16(Frag<bf16_t>& f, uint32_t lo, uint32_t hi) {
  f.set_pair(0, e4m3_byte<0>(lo), e4m3_byte<1>(lo));
  f.set_pair(1, e4m3_byte<2>(lo), e4m3_byte<3>(lo));
  f.set_pair(2, e4m3_byte<0>(hi), e4m3_byte<1>(hi));
  f.set_pair(3, e4m3_byte<2>(hi), e4m3_byte<3>(hi));
}


// Readout of the linear branch for NQ blocks of 16 queries (one fragment
// column each): phi_q = elu(q U_q) + 1, q' = rope(phi_q),
// O_lW = (q' S') / (phi_q . z).  Every U_q^T and S' fragment is fetched once
// and used for all NQ blocks.  qf[b] holds block b's queries as B fragments;
// results land in the accumulator layout of O^T (lane: query l%16, dims
// 16 jd + 4 (l/16) + i).
template <typename T, int D, int R, int NQ>
__device__ __forceinline__ void readout(const ReadoutSrc<T>& a, const Frag<T> (*qf)[D / 32], const int* qrow,
                                        const bool* qvalid, int lane, f32x4 (*acc_n)[D / 16], float* inv_den,
                                        float qscale = 1.f) {
  constexpr int NDB = D / 16;
  constexpr int NRB = R / 16;
  constexpr int NRC = (R + 31) / 32;
  const int g = lane >> 4;
  const T* UQ = a.uq;
  const float* Z = a.z;
  f32x4 f[NQ][NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
    for (int b = 0; b < NQ; ++b) f[b][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      Frag<T> uf;
      load8(uf, UQ + ((size_t)(rb * (D / 32) + c) * 64 + lane) * 8);
#pragma unroll
      for (int b = 0; b < NQ; ++b) mma(f[b][rb], uf, qf[b][c]);
    }
  }
  const int ht = 3 * R / 16, hh = 3 * R / 16, hwp = R / 8;
  Frag<T> qpf[NQ][NRC];
#pragma unroll
  for (int b = 0; b < NQ; ++b) {
    int qpos[3];
    {
      const int tok = qvalid[b] ? qrow[b] : 0, hw = a.gh * a.gw;
      qpos[0] = tok / hw;
      const int rem = tok - qpos[0] * hw;
      qpos[1] = rem / a.gw;
      qpos[2] = rem - qpos[1] * a.gw;
    }
    float den = 0.f;
    float qp[NRB][4];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float phi = elu1(f[b][rb][i] * qscale);  // qscale: fp8 tile scale of the queries
        f[b][rb][i] = phi;
        den += phi * Z[16 * rb + 4 * g + i];
      }
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const int jp = (16 * rb + 4 * g) / 2 + pr;
        int axis, m, half, off;
        if (jp < ht) { axis = 0; m = jp; half = ht; off = 0; }
        else if (jp < ht + hh) { axis = 1; m = jp - ht; half = hh; off = a.gt * ht; }
        else { axis = 2; m = jp - ht - hh; half = hwp; off = a.gt * ht + a.gh * hh; }
        const float2 cs = a.rope[off + qpos[axis] * half + m];
        const float x0 = f[b][rb][2 * pr], x1 = f[b][rb][2 * pr + 1];
        qp[rb][2 * pr] = x0 * cs.x - x1 * cs.y;
        qp[rb][2 * pr + 1] = x0 * cs.y + x1 * cs.x;
      }
    }
    den = group4_sum(den);
    inv_den[b] = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
    for (int rc = 0; rc < NRC; ++rc) {
      constexpr int kHi = 1;  // second 16-block of the 32-wide chunk
      const int b0 = 2 * rc, b1 = (2 * rc + kHi < NRB) ? 2 * rc + kHi : 2 * rc;
      const float keep = (2 * rc + kHi < NRB) ? 1.f : 0.f;  // rank 16: upper half is zero
      qpf[b][rc].set_pair(0, qp[b0][0], qp[b0][1]);
      qpf[b][rc].set_pair(1, qp[b0][2], qp[b0][3]);
      qpf[b][rc].set_pair(2, keep * qp[b1][0], keep * qp[b1][1]);
      qpf[b][rc].set_pair(3, keep * qp[b1][2], keep * qp[b1][3]);
    }
  }
  constexpr int NFE = NDB * NRC * 512;
  const T* SP = a.sp;
#pragma unroll
  for (int jd = 0; jd < NDB; ++jd) {
#pragma unroll
    for (int b = 0; b < NQ; ++b) acc_n[b][jd] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rc = 0; rc < NRC; ++rc) {
      Frag<T> sf;
      load8(sf, SP + ((size_t)(jd * NRC + rc) * 64 + lane) * 8);
#pragma unroll
      for (int b = 0; b < NQ; ++b) mma(acc_n[b][jd], sf, qpf[b][rc]);
      if constexpr (sizeof(T) == 2) {
        load8(sf, SP + NFE + ((size_t)(jd * NRC + rc) * 64 + lane) * 8);
#pragma unroll
        for (int b = 0; b < NQ; ++b) mma(acc_n[b][jd], sf, qpf[b][rc]);
      }
    }
  }
}

}  // namespace hsa
