// Query-tile kernel: block-sparse flash attention over the kept key tiles,
// followed by the readout of the rotary low-rank linear branch, both summed in
// one epilogue (SparkDiffusion news article, section 05: the sparse branch
// keeps the high-energy tile interactions, the linear branch restores the
// global context).
//
// One block = one (b, h, query tile) = 64 queries, 4 waves of 16 queries.
// Scores are formed transposed, S^T = K Q^T, so that each lane owns one query
// column: the softmax max/sum run mostly in-lane, and the score accumulator
// already sits in the operand layout of P^T for O^T += V^T P^T.  K tiles are
// staged row-major in LDS; V tiles transposed, with keys permuted inside
// every 32-key chunk to match that operand layout.  Two LDS stages and a
// register prefetch overlap the next tile's HBM/L2 reads with the current
// tile's matrix-core work.
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace hsa {

struct AttendArgs {
  int N, N_pad, T, H;
  int gt, gh, gw;
  float scale_log2;  // softmax scale * log2(e)
  const void* q;
  const void* k;
  const void* v;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const void* sp_frag;
  const float* z;
  const void* uq_frag;
  const float2* rope;
  void* o;
  float* lse;
  long nrows;
};

__device__ __forceinline__ int vt_pos_a(int key) {
  int c = key >> 5, kk = key & 31;
  int h = kk >> 4, g = (kk >> 2) & 3, i = kk & 3;
  return 32 * c + 8 * g + 4 * h + i;
}

__device__ __forceinline__ void st4o(bf16_t* dst, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}
__device__ __forceinline__ void st4o(float* dst, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void st4v(bf16_t* dst, float a, float b, float c, float d) { st4o(dst, a, b, c, d); }
__device__ __forceinline__ void st4v(float* dst, float a, float b, float c, float d) { st4o(dst, a, b, c, d); }

__device__ __forceinline__ void lds_row(bf16_t* dst, const Chunk8<bf16_t>& c) { *reinterpret_cast<u32x4*>(dst) = c.w; }
__device__ __forceinline__ void lds_row(float* dst, const Chunk8<float>& c) {
  reinterpret_cast<float4*>(dst)[0] = c.a;
  reinterpret_cast<float4*>(dst)[1] = c.b;
}

template <typename T, int D, int R, bool SPARSE, bool LINEAR>
__global__ __launch_bounds__(256, 2) void k_attend(AttendArgs a) {
  constexpr int CPR = D / 8;
  constexpr int NCONT = 256 / CPR;
  constexpr int KCH = 64 * CPR / 256;
  constexpr int NVU = 16 * CPR;
  constexpr int KSTR = D + 8;
  constexpr int VSTR = 64 + 8;
  constexpr int NDB = D / 16;
  constexpr int NRB = R / 16;
  constexpr int NRC = (R + 31) / 32;
  constexpr int STAGE = SPARSE ? (64 * KSTR + D * VSTR) : 1;
  __shared__ __align__(16) T lds[2 * STAGE];

  const long L = xcd_remap(blockIdx.x, a.nrows);
  if (L < 0) return;
  const int bh = (int)(L / a.T), qa = (int)(L % a.T);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const size_t base = (size_t)bh * a.N_pad * D;
  const T* Q = reinterpret_cast<const T*>(a.q) + base;
  const T* K = reinterpret_cast<const T*>(a.k) + base;
  const T* V = reinterpret_cast<const T*>(a.v) + base;
  const int qrow = qa * 64 + 16 * w + l16;  // this lane's query
  const bool qvalid = qrow < a.N;

  Frag<T> qf[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    if (qvalid) load8(qf[c], Q + (size_t)qrow * D + 32 * c + 8 * g);
    else qf[c].zero();
  }

  f32x4 acc_o[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j) acc_o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float inv_l = 0.f;

  if constexpr (SPARSE) {
    const int beg = a.row_ptr[(size_t)bh * a.T + qa];
    const int end = a.row_ptr[(size_t)bh * a.T + qa + 1];
    float m = -INFINITY, lsum = 0.f;
    const int col8 = tid % CPR, row0 = tid / CPR;
    Chunk8<T> kc[KCH], vc[4];
    auto load_tile = [&](int col) {
      const bool ok = col >= 0 && col < a.T;
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        int gr = col * 64 + row0 + i * NCONT;
        if (ok && gr < a.N) gload8(kc[i], K + (size_t)gr * D + col8 * 8);
        else zero8(kc[i]);
      }
      if (tid < NVU) {
        int kg = tid % 16, c8 = tid / 16;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          int gr = col * 64 + 4 * kg + ii;
          if (ok && gr < a.N) gload8(vc[ii], V + (size_t)gr * D + c8 * 8);
          else zero8(vc[ii]);
        }
      }
    };
    if (beg < end) load_tile(a.col_idx[beg]);
    for (int j = beg; j < end; ++j) {
      T* Ks = lds + ((j - beg) & 1) * STAGE;
      T* Vt = Ks + 64 * KSTR;
      const int col = a.col_idx[j];
#pragma unroll
      for (int i = 0; i < KCH; ++i) lds_row(&Ks[(row0 + i * NCONT) * KSTR + col8 * 8], kc[i]);
      if (tid < NVU) {
        int kg = tid % 16, c8 = tid / 16;
        int p0 = vt_pos_a(4 * kg);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          st4v(&Vt[(c8 * 8 + e) * VSTR + p0], elem(vc[0], e), elem(vc[1], e), elem(vc[2], e), elem(vc[3], e));
      }
      __syncthreads();
      if (j + 1 < end) load_tile(a.col_idx[j + 1]);

      const int kvalid = (col >= 0 && col < a.T) ? min(64, a.N - col * 64) : 0;
      f32x4 s[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          Frag<T> kf;
          load8(kf, &Ks[(16 * kb + l16) * KSTR + 32 * c + 8 * g]);
          mma(s[kb], kf, qf[c]);
        }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = (16 * kb + 4 * g + i < kvalid) ? s[kb][i] * a.scale_log2 : -INFINITY;
          s[kb][i] = x;
          mt = fmaxf(mt, x);
        }
      mt = group4_max(mt);
      const float mn = fmaxf(m, mt);
      const bool dead = (mn == -INFINITY);
      const float alpha = dead ? 1.f : exp2f(m - mn);
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float p = dead ? 0.f : exp2f(s[kb][i] - mn);
          s[kb][i] = p;
          ps += p;
        }
      lsum = lsum * alpha + ps;
      m = mn;
#pragma unroll
      for (int jd = 0; jd < NDB; ++jd) acc_o[jd] *= alpha;
      Frag<T> pf[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        pf[c].set_pair(0, s[2 * c][0], s[2 * c][1]);
        pf[c].set_pair(1, s[2 * c][2], s[2 * c][3]);
        pf[c].set_pair(2, s[2 * c + 1][0], s[2 * c + 1][1]);
        pf[c].set_pair(3, s[2 * c + 1][2], s[2 * c + 1][3]);
      }
#pragma unroll
      for (int jd = 0; jd < NDB; ++jd)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          Frag<T> vf;
          load8(vf, &Vt[(16 * jd + l16) * VSTR + 32 * c + 8 * g]);
          mma(acc_o[jd], vf, pf[c]);
        }
    }
    const float lt = group4_sum(lsum);
    inv_l = lt > 0.f ? 1.f / lt : 0.f;
    if (a.lse && g == 0 && qvalid) a.lse[(size_t)bh * a.N_pad + qrow] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
  }

  f32x4 acc_n[NDB];
  float inv_den = 0.f;
  if constexpr (LINEAR) {
    const int h = bh % a.H;
    const T* UQ = reinterpret_cast<const T*>(a.uq_frag) + (size_t)h * NRB * (D / 32) * 512;
    const float* Z = a.z + (size_t)bh * R;
    f32x4 f[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      f[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        Frag<T> uf;
        load8(uf, UQ + ((size_t)(rb * (D / 32) + c) * 64 + lane) * 8);
        mma(f[rb], uf, qf[c]);
      }
    }
    // query position
    int qpos[3];
    {
      int tok = qvalid ? qrow : 0, hw = a.gh * a.gw;
      qpos[0] = tok / hw;
      int rem = tok - qpos[0] * hw;
      qpos[1] = rem / a.gw;
      qpos[2] = rem - qpos[1] * a.gw;
    }
    const int ht = 3 * R / 16, hh = 3 * R / 16, hwp = R / 8;
    float den = 0.f;
    float qp[NRB][4];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float phi = elu1(f[rb][i]);
        f[rb][i] = phi;
        den += phi * Z[16 * rb + 4 * g + i];
      }
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        int jp = (16 * rb + 4 * g) / 2 + pr;
        int axis, m, half, off;
        if (jp < ht) { axis = 0; m = jp; half = ht; off = 0; }
        else if (jp < ht + hh) { axis = 1; m = jp - ht; half = hh; off = a.gt * ht; }
        else { axis = 2; m = jp - ht - hh; half = hwp; off = a.gt * ht + a.gh * hh; }
        float2 cs = a.rope[off + qpos[axis] * half + m];
        float x0 = f[rb][2 * pr], x1 = f[rb][2 * pr + 1];
        qp[rb][2 * pr] = x0 * cs.x - x1 * cs.y;
        qp[rb][2 * pr + 1] = x0 * cs.y + x1 * cs.x;
      }
    }
    den = group4_sum(den);
    inv_den = den > 0.f ? 1.f / den : 0.f;
    Frag<T> qpf[NRC];
#pragma unroll
    for (int rc = 0; rc < NRC; ++rc) {
      constexpr int kHi = 1;  // second 16-block of the 32-wide chunk
      const int b0 = 2 * rc, b1 = (2 * rc + kHi < NRB) ? 2 * rc + kHi : 2 * rc;
      const float keep = (2 * rc + kHi < NRB) ? 1.f : 0.f;  // rank 16: upper half is zero
      qpf[rc].set_pair(0, qp[b0][0], qp[b0][1]);
      qpf[rc].set_pair(1, qp[b0][2], qp[b0][3]);
      qpf[rc].set_pair(2, keep * qp[b1][0], keep * qp[b1][1]);
      qpf[rc].set_pair(3, keep * qp[b1][2], keep * qp[b1][3]);
    }
    constexpr int NFE = NDB * NRC * 512;
    const T* SP = reinterpret_cast<const T*>(a.sp_frag) + (size_t)bh * (sizeof(T) == 4 ? 1 : 2) * NFE;
#pragma unroll
    for (int jd = 0; jd < NDB; ++jd) {
      acc_n[jd] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int rc = 0; rc < NRC; ++rc) {
        Frag<T> sf;
        load8(sf, SP + ((size_t)(jd * NRC + rc) * 64 + lane) * 8);
        mma(acc_n[jd], sf, qpf[rc]);
        if constexpr (sizeof(T) == 2) {
          load8(sf, SP + NFE + ((size_t)(jd * NRC + rc) * 64 + lane) * 8);
          mma(acc_n[jd], sf, qpf[rc]);
        }
      }
    }
  }

  // epilogue: O = O_s / l + (q' S') / den, pad rows zero
  T* O = reinterpret_cast<T*>(a.o) + base + (size_t)qrow * D;
  if (qrow < a.N_pad) {
#pragma unroll
    for (int jd = 0; jd < NDB; ++jd) {
      float r4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = 0.f;
        if constexpr (SPARSE) x += acc_o[jd][i] * inv_l;
        if constexpr (LINEAR) x += acc_n[jd][i] * inv_den;
        r4[i] = qvalid ? x : 0.f;
      }
      st4o(O + 16 * jd + 4 * g, r4[0], r4[1], r4[2], r4[3]);
    }
  }
}

// Launch helpers shared by the bf16/fp8 translation unit and the float32 one.
template <typename T, int D, int R>
static hipError_t attend_dispatch(const AttendArgs& a, bool sparse, bool linear, hipStream_t st) {
  const long grid = 8 * ((a.nrows + 7) / 8);
  if (sparse && linear) k_attend<T, D, R, true, true><<<grid, 256, 0, st>>>(a);
  else if (sparse) k_attend<T, D, R, true, false><<<grid, 256, 0, st>>>(a);
  else k_attend<T, D, R, false, true><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <typename T>
static hipError_t attend_by_shape(const Shape& s, const AttendArgs& a, bool sparse, bool linear, hipStream_t st) {
  if (!linear) return s.d == 64 ? attend_dispatch<T, 64, 16>(a, sparse, linear, st)
                                : attend_dispatch<T, 128, 16>(a, sparse, linear, st);
  if (s.d == 64) {
    if (s.rank == 16) return attend_dispatch<T, 64, 16>(a, sparse, linear, st);
    if (s.rank == 32) return attend_dispatch<T, 64, 32>(a, sparse, linear, st);
    return attend_dispatch<T, 64, 64>(a, sparse, linear, st);
  }
  if (s.rank == 16) return attend_dispatch<T, 128, 16>(a, sparse, linear, st);
  if (s.rank == 32) return attend_dispatch<T, 128, 32>(a, sparse, linear, st);
  return attend_dispatch<T, 128, 64>(a, sparse, linear, st);
}

hipError_t launch_attend_f32(const Shape& s, const AttendArgs& a, bool sparse, bool linear, hipStream_t st);

}  // namespace hsa
