// Query-tile kernels: block-sparse flash attention over the kept key tiles,
// followed by the readout of the rotary low-rank linear branch, both summed in
// one epilogue (SparkDiffusion news article, section 05: the sparse branch
// keeps the high-energy tile interactions, the linear branch restores the
// global context).
//
// Common to all three kernels: scores are formed transposed, S^T = K Q^T, so
// that each lane owns one query column (the softmax max and sum run mostly
// in-lane) and the score accumulator already sits in the operand layout of P^T
// for O^T += V^T P^T.
//  * k_attend<float>: the float32 kernel (4 waves of 16 queries, K staged
//    row-major and V transposed in LDS, two stages).
//  * k_attend_bf16: 2 waves of 32 queries, K/V tiles moved global -> LDS by
//    LDS-direct loads into XOR-swizzled tiles, V operands by transposing reads.
//  * k_attend_fp8: the same staging over pairs of kept tiles, 16x16x128 fp8
//    matrix-core steps, per-tile scales folded into the exp2 argument.
#pragma once

#include <type_traits>
#include <stdlib.h>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_dma.hpp"
#include "readout.hpp"

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
  const void* vt;  // fp8 path: V tiles transposed ([BH][T][d][64] codes, keys permuted)
  const float* qs;  // fp8 path: per-(b, h, tile) scales of Q, K, V
  const float* ks;
  const float* vs;
  void* o;
  float* lse;
  void* o_s;  // optional, sparse + linear kernels of bf16/float inputs: O_s alone (output type, rows >= N zero)
  long nrows;
};

// Readout operands of (b, h) from the finalized state in the workspace.
template <typename T, int D, int R>
__device__ __forceinline__ ReadoutSrc<T> readout_src(const AttendArgs& a, int bh) {
  constexpr int NRB = R / 16, NRC = (R + 31) / 32, NFE = (D / 16) * NRC * 512;
  ReadoutSrc<T> s;
  s.uq = reinterpret_cast<const T*>(a.uq_frag) + (size_t)(bh % a.H) * NRB * (D / 32) * 512;
  s.sp = reinterpret_cast<const T*>(a.sp_frag) + (size_t)bh * (sizeof(T) == 4 ? 1 : 2) * NFE;
  s.z = a.z + (size_t)bh * R;
  s.rope = a.rope;
  s.gt = a.gt; s.gh = a.gh; s.gw = a.gw;
  return s;
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

  const int L = uniform(head_interleaved_row(blockIdx.x, a.T));
  if (L < 0) return;
  const int bh = uniform(L / a.T), qa = uniform(L - bh * a.T);
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

  f32x4 acc_n[1][NDB];
  float inv_den[1] = {0.f};
  if constexpr (LINEAR) {
    const int qr[1] = {qrow};
    const bool qv[1] = {qvalid};
    readout<T, D, R, 1>(readout_src<T, D, R>(a, bh), &qf, qr, qv, lane, acc_n, inv_den);
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
        if constexpr (LINEAR) x += acc_n[0][jd][i] * inv_den[0];
        r4[i] = qvalid ? x : 0.f;
      }
      st4o(O + 16 * jd + 4 * g, r4[0], r4[1], r4[2], r4[3]);
    }
    if constexpr (SPARSE && LINEAR) {
      if (a.o_s) {  // the sparse branch's output alone, as the sparse-only kernel writes it
        T* OS = reinterpret_cast<T*>(a.o_s) + base + (size_t)qrow * D;
#pragma unroll
        for (int jd = 0; jd < NDB; ++jd) {
          float r4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x = 0.f;
            x += acc_o[jd][i] * inv_l;
            r4[i] = qvalid ? x : 0.f;
          }
          st4o(OS + 16 * jd + 4 * g, r4[0], r4[1], r4[2], r4[3]);
        }
      }
    }
  }
}


// Row maxima of raw scores.  fmaxf on values the compiler cannot prove
// canonical (matrix-core results) costs one extra canonicalizing v_max per
// input under IEEE mode; the IEEE 754-2019 maximum lowers to v_maximum3_f32
// with none.  The two differ only for NaN and signed zero, and a score is
// never NaN (masked keys are -inf, where both agree).
__device__ __forceinline__ float smax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float smax4(const f32x4& v) { return smax(smax(v[0], v[1]), smax(v[2], v[3])); }

// ---------------------------------------------------------------------------
// bf16 query-tile kernel.  One block = one (b, h, query tile) = 2 waves of 32
// queries; each wave keeps its queries as two 16-column B-fragment sets, so
// every K or V fragment read from LDS feeds two matrix-core steps.
//
// Staging.  Key tiles travel global -> LDS by buffer loads that write LDS
// directly (no registers in between): one such load moves 64 lanes x 16 bytes
// into 1 KB of contiguous LDS, lane l at byte 16 l.  K and V have one LDS
// buffer each; the loads of the next K tile are issued once both waves are
// done with the current one (after the scores), those of the next V tile once
// both are done with the PV step, so each load has about half an iteration to
// land.  A tile index outside [0, T) reads as zeros and is skipped.
//
// Layout.  Rows are stored unpadded, their 16-byte granules permuted by an
// XOR swizzle (position = granule ^ f(row)) so that fragment reads are free
// of bank conflicts: for K, the 16 rows of a 16-byte fragment read land on 16
// distinct granule positions of the 64 banks; for V, each half wave of a
// transposing 8-byte read touches 8 rows x 32 bytes, 8 distinct granule pairs.
// V fragments come straight from the row-major tile through
// ds_read_b64_tr_b16: within each 16-lane group, output lane i, element t is
// element (i mod 4) of the 8 bytes addressed by source lane 4t + i/4.
// ---------------------------------------------------------------------------
template <int D, int R, bool SPARSE, bool LINEAR>
__global__ __launch_bounds__(128, 2) void k_attend_bf16(AttendArgs a) {
  constexpr int RB = 2 * D, RG = RB / 16;  // bytes and granules per row
  constexpr int NQB = 2;                   // 16-query blocks per wave
  constexpr int NDB = D / 16;
  constexpr int NI = 64 * RB / 1024 / 2;   // LDS-direct loads per wave per tile
  __shared__ __align__(16) uint8_t Ks[SPARSE ? 64 * RB : 16];
  __shared__ __align__(16) uint8_t Vs[SPARSE ? 64 * RB : 16];

  const int L = uniform(head_interleaved_row(blockIdx.x, a.T));
  if (L < 0) return;
  const int bh = uniform(L / a.T), qa = uniform(L - bh * a.T);
  const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const size_t base = (size_t)bh * a.N_pad * D;
  const bf16_t* Q = reinterpret_cast<const bf16_t*>(a.q) + base;
  const bf16_t* K = reinterpret_cast<const bf16_t*>(a.k) + base;
  const bf16_t* V = reinterpret_cast<const bf16_t*>(a.v) + base;

  // Bounds-checked buffer views of this head: rows >= N read as zero, and so
  // does any offset past the slice (an out-of-range tile index included).
  const int nbytes = a.N * RB;
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc((void*)Q, 0, nbytes, kBufferFlags);
  const i32x4_t krs = make_rsrc_regs(K, nbytes);
  const i32x4_t vrs = make_rsrc_regs(V, nbytes);

  int qrow[NQB];
  bool qvalid[NQB];
  Frag<bf16_t> qf[NQB][D / 32];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    qrow[qb] = qa * 64 + 32 * w + 16 * qb + l16;
    qvalid[qb] = qrow[qb] < a.N;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      qf[qb][c].w = __builtin_amdgcn_raw_buffer_load_b128(qrs, (qrow[qb] * D + 32 * c + 8 * g) * 2, 0, 0);
  }

  f32x4 acc_o[NQB][NDB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int j = 0; j < NDB; ++j) acc_o[qb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float inv_l[NQB] = {0.f, 0.f};

  if constexpr (SPARSE) {
    // The LDS tiles are only written by the LDS-direct loads, which the
    // compiler does not see; this store, never executed, keeps it from
    // treating them as unwritten.
    if (a.N < 0) { Ks[tid] = 0; Vs[tid] = 0; }
    const int beg = a.row_ptr[(size_t)bh * a.T + qa];
    const int end = a.row_ptr[(size_t)bh * a.T + qa + 1];
    // Running max (log2 units) is only raised when a row's new max exceeds
    // it by more than 8, so exp2 arguments stay <= 8 and most tiles skip the
    // rescale of O; the final O / l is the same for any valid max.
    float m[NQB] = {-INFINITY, -INFINITY};
    f32x4 acc_l[NQB];  // row sums of P, formed on the matrix cores
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) acc_l[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    Frag<bf16_t> ones;
    ones.w = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const float c2 = a.scale_log2;
    int koff[NI], voff[NI];
    dma_offsets<RB, false>(w, lane, koff);
    dma_offsets<RB, true>(w, lane, voff);
    // fragment read addresses: K (16 B) per 32-wide d chunk cc; V (8 B, transposing) per 16-wide d block jd
    const int fk = swz_k<RG>(l16);
    const int kaddr = l16 * RB + 16 * (g ^ fk);                   // ^ 64 cc, + 16 RB kb
    const int rowl = 4 * g + (l16 >> 2);
    const int vaddr = rowl * RB + 16 * swz_v<RG>(rowl) + 16 * ((l16 >> 1) & 1) + 8 * (l16 & 1);  // ^ 32 jd
    // The row's tile indices, 64 at a time, one per lane: the loop reads them
    // with readlane; col / ncol are the indices of tiles j and j + 1.
    int colv = beg + lane < end ? a.col_idx[beg + lane] : 0;
    int col = __builtin_amdgcn_readlane(colv, 0);
    int ncol = __builtin_amdgcn_readlane(colv, 1);
    if (beg < end) {
      dma_tile<RB>(krs, col, koff, Ks, w);
      dma_tile<RB>(vrs, col, voff, Vs, w);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(NI));  // this wave's K share has landed
      __syncthreads();
    }
    for (int j = beg; j < end; ++j) {
      const bool more = j + 1 < end;
      const int kvalid = (col >= 0 && col < a.T) ? min(64, a.N - col * 64) : 0;
      Frag<bf16_t> pf[NQB][2];
      f32x4 s[NQB][4];
      if (kvalid > 0) {
        // S^T = K Q^T: 4 key blocks x 2 query blocks (raw scores); the K
        // fragments of key block kb + 1 are read while kb's steps run
        Frag<bf16_t> kf[2][D / 32];
        auto ldk = [&](int kb, Frag<bf16_t>* dst) {
#pragma unroll
          for (int c = 0; c < D / 32; ++c)
            dst[c].w = *reinterpret_cast<const u32x4*>(&Ks[(kaddr ^ (64 * c)) + 16 * RB * kb]);
        };
        ldk(0, kf[0]);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          if (kb + 1 < 4) ldk(kb + 1, kf[(kb + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) s[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < D / 32; ++c)
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) mma(s[qb][kb], kf[kb & 1][c], qf[qb][c]);
        }
        if (__builtin_expect(kvalid < 64, 0)) {  // ragged last tile: keys past N do not exist
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (16 * kb + 4 * g + i >= kvalid) s[qb][kb][i] = -INFINITY;
        }
        // The common path needs no cross-lane work: if no lane's own keys exceed
        // the running max by more than 8, every exp2 argument is <= 8.
        float mloc[NQB];
        bool raise = false;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const float mx = smax(smax(smax4(s[qb][0]), smax4(s[qb][1])), smax(smax4(s[qb][2]), smax4(s[qb][3])));
          mloc[qb] = mx * c2;
          raise |= mloc[qb] > m[qb] + 8.f;
        }
        if (__ballot(raise)) {
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) {
            const float mt = group4_max(mloc[qb]);  // the row max, the same in all four lane groups
            const float mn = mt > m[qb] + 8.f ? fmaxf(m[qb], mt) : m[qb];
            const float alpha = __builtin_amdgcn_exp2f(m[qb] - mn);
            m[qb] = mn;
#pragma unroll
            for (int jd = 0; jd < NDB; ++jd) acc_o[qb][jd] *= alpha;
            acc_l[qb] *= alpha;
          }
        }
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const float nm = -m[qb];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) s[qb][kb][i] = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][i], c2, nm));
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            pf[qb][c].set_pair(0, s[qb][2 * c][0], s[qb][2 * c][1]);
            pf[qb][c].set_pair(1, s[qb][2 * c][2], s[qb][2 * c][3]);
            pf[qb][c].set_pair(2, s[qb][2 * c + 1][0], s[qb][2 * c + 1][1]);
            pf[qb][c].set_pair(3, s[qb][2 * c + 1][2], s[qb][2 * c + 1][3]);
            mma(acc_l[qb], ones, pf[qb][c]);
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // this wave's V share has landed
      lds_barrier();                              // V visible; both waves are done with K
      if (more) dma_tile<RB>(krs, ncol, koff, Ks, w);  // the next K tile loads during the PV step
      if (kvalid > 0) {
        // O^T += V^T P^T; slot s of lane group g holds key 32c + 16(s/4) + 4g + s%4.
        // The V fragments of d block jd + 1 are read while jd's steps run.
        Frag<bf16_t> vf[2][2];
        auto ldv = [&](int jd, Frag<bf16_t>* dst) {
          const int va = vaddr ^ (32 * jd);
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const uint8_t* src = &Vs[va + (32 * c + 16 * hh) * RB];
              s16x4_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(src));
              uint2 u = __builtin_bit_cast(uint2, t);
              dst[c].w[2 * hh] = u.x;
              dst[c].w[2 * hh + 1] = u.y;
            }
        };
        ldv(0, vf[0]);
#pragma unroll
        for (int jd = 0; jd < NDB; ++jd) {
          if (jd + 1 < NDB) ldv(jd + 1, vf[(jd + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the steps that do not need them
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) mma(acc_o[qb][jd], vf[jd & 1][c], pf[qb][c]);
        }
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // this wave's share of the next K has landed
      lds_barrier();                              // next K visible; both waves are done with V
      if (((j + 2 - beg) & 63) == 0 && j + 2 < end) {
        // the next 64 indices; nothing else is in flight at this point
        colv = j + 2 + lane < end ? a.col_idx[j + 2 + lane] : 0;
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      }
      if (more) dma_tile<RB>(vrs, ncol, voff, Vs, w);
      col = ncol;
      ncol = __builtin_amdgcn_readlane(colv, (j + 2 - beg) & 63);
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const float lt = acc_l[qb][0];  // every row of the ones product holds the sum
      inv_l[qb] = lt > 0.f ? 1.f / lt : 0.f;
      if (a.lse && g == 0 && qvalid[qb])
        a.lse[(size_t)bh * a.N_pad + qrow[qb]] = lt > 0.f ? (m[qb] + __log2f(lt)) * kLn2 : -INFINITY;
    }
  }

  f32x4 acc_n[NQB][NDB];
  float inv_den[NQB] = {0.f, 0.f};
  if constexpr (LINEAR) readout<bf16_t, D, R, NQB>(readout_src<bf16_t, D, R>(a, bh), qf, qrow, qvalid, lane, acc_n, inv_den);
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    bf16_t* O = reinterpret_cast<bf16_t*>(a.o) + base + (size_t)qrow[qb] * D;
#pragma unroll
    for (int jd = 0; jd < NDB; ++jd) {
      float r4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = 0.f;
        if constexpr (SPARSE) x += acc_o[qb][jd][i] * inv_l[qb];
        if constexpr (LINEAR) x += acc_n[qb][jd][i] * inv_den[qb];
        r4[i] = qvalid[qb] ? x : 0.f;
      }
      st4o(O + 16 * jd + 4 * g, r4[0], r4[1], r4[2], r4[3]);
    }
  }
  if constexpr (SPARSE && LINEAR) {
    if (a.o_s) {  // the sparse branch's output alone, as the sparse-only kernel writes it
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        bf16_t* OS = reinterpret_cast<bf16_t*>(a.o_s) + base + (size_t)qrow[qb] * D;
#pragma unroll
        for (int jd = 0; jd < NDB; ++jd) {
          float r4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x = 0.f;
            x += acc_o[qb][jd][i] * inv_l[qb];
            r4[i] = qvalid[qb] ? x : 0.f;
          }
          st4o(OS + 16 * jd + 4 * g, r4[0], r4[1], r4[2], r4[3]);
        }
      }
    }
  }
}

template <int D, int R>
static hipError_t attend_dispatch_bf16(const AttendArgs& a, bool sparse, bool linear, hipStream_t st) {
  const long grid = 8 * (a.nrows / a.T) * ((a.T + 7) / 8);
  if (sparse && linear) k_attend_bf16<D, R, true, true><<<grid, 128, 0, st>>>(a);
  else if (sparse) k_attend_bf16<D, R, true, false><<<grid, 128, 0, st>>>(a);
  else k_attend_bf16<D, R, false, true><<<grid, 128, 0, st>>>(a);
  return hipGetLastError();
}

static inline hipError_t attend_bf16_by_shape(const Shape& s, const AttendArgs& a, bool sparse, bool linear,
                                              hipStream_t st) {
  if (!linear) return s.d == 64 ? attend_dispatch_bf16<64, 16>(a, sparse, linear, st)
                                : attend_dispatch_bf16<128, 16>(a, sparse, linear, st);
  if (s.d == 64) {
    if (s.rank == 16) return attend_dispatch_bf16<64, 16>(a, sparse, linear, st);
    if (s.rank == 32) return attend_dispatch_bf16<64, 32>(a, sparse, linear, st);
    return attend_dispatch_bf16<64, 64>(a, sparse, linear, st);
  }
  if (s.rank == 16) return attend_dispatch_bf16<128, 16>(a, sparse, linear, st);
  if (s.rank == 32) return attend_dispatch_bf16<128, 32>(a, sparse, linear, st);
  return attend_dispatch_bf16<128, 64>(a, sparse, linear, st);
}

// ---------------------------------------------------------------------------
// fp8 query-tile kernel (OCP E4M3FN codes with one fp32 scale per
// (b, h, 64-token tile, tensor)).  One block = one query tile = 2 waves of 32
// queries, d = 128.  Kept key tiles are taken in pairs so that one
// 16x16x128 fp8 matrix-core step contracts over 128 keys:
//   S = (q8 . k8) * s_q * s_k       (the scales enter the exp2 multiplier)
//   P'_k = fp8(P_k * s_v,t / s_v,ref)   (s_v,ref: largest V scale of the
//                                    row's kept tiles, so P' <= 256)
//   O = s_v,ref * sum_k P'_k v8_k / sum_k P'_k s_v,ref / s_v,t
// The denominator uses the same rounded P' as the numerator (its per-tile
// sums come from a matrix-core step against a ones operand), so O is an
// exact convex combination of the V rows with weights P'_k s_v,ref / s_v,t.
// V tiles arrive transposed from the streaming pass (d rows of 64 key codes,
// keys ordered so that lane group g reads its 16 keys of a tile as one
// 16-byte granule).  Staging, buffers and barriers follow the bf16 kernel:
// LDS-direct loads into XOR-swizzled unpadded tiles, the next K pair loading
// during the PV step and the next V pair during the score step.
// ---------------------------------------------------------------------------
// Swizzles of the fp8 tiles (K rows of 128 bytes, V^T rows of 64 bytes):
// granule p of row r sits at position p ^ f(r).  The rule by which gfx950
// serves the lanes of a 16-byte LDS read was measured, not assumed: with the
// LDS bank-conflict counter, a probe over every XOR swizzle of the K rows
// linear in the row bits reads 0 conflict cycles for the one below and 4 per
// read instruction for f(r) = r & 7 or (r >> 1) & 7; for the V^T rows,
// (r >> 1) & 3 reads 0 and (r >> 2) & 3 reads 4.
__device__ __forceinline__ int swz_k8(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }
__device__ __forceinline__ int swz_v8(int row) { return (row >> 1) & 3; }

template <int R, bool SPARSE, bool LINEAR>
__global__ __launch_bounds__(128, 2) void k_attend_fp8(AttendArgs a) {
  constexpr int D = 128;
  constexpr int NQB = 2;
  constexpr int NDB = D / 16;
  constexpr int KT = 64 * D;       // bytes of one K tile (64 rows x 128 codes)
  constexpr int VT = D * 64;       // bytes of one V^T tile (128 rows x 64 codes)
  constexpr int NI = 2 * KT / 1024 / 2;  // LDS-direct loads per wave per pair (K; the same for V)
  __shared__ __align__(16) uint8_t Ks[SPARSE ? 2 * KT : 16];
  __shared__ __align__(16) uint8_t Vs[SPARSE ? 2 * VT : 16];

  const int L = uniform(head_interleaved_row(blockIdx.x, a.T));
  if (L < 0) return;
  const int bh = uniform(L / a.T), qa = uniform(L - bh * a.T);
  const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const size_t base = (size_t)bh * a.N_pad * D;
  const uint8_t* Q = reinterpret_cast<const uint8_t*>(a.q) + base;
  const uint8_t* K = reinterpret_cast<const uint8_t*>(a.k) + base;
  const uint8_t* VT8 = reinterpret_cast<const uint8_t*>(a.vt) + base;  // T*64*D codes per head
  const int nbytes = a.N * D;
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc((void*)Q, 0, nbytes, kBufferFlags);
  const i32x4_t krs = make_rsrc_regs(K, nbytes);
  const i32x4_t vrs = make_rsrc_regs(VT8, a.T * VT);
  const float* SQ = a.qs + (size_t)bh * a.T;
  const float* SK = a.ks + (size_t)bh * a.T;
  const float* SV = a.vs + (size_t)bh * a.T;
  const float sq = SQ[qa];

  int qrow[NQB];
  bool qvalid[NQB];
  i32x8_t qf8[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    qrow[qb] = qa * 64 + 32 * w + 16 * qb + l16;
    qvalid[qb] = qrow[qb] < a.N;
    const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(qrs, qrow[qb] * D + 32 * g, 0, 0);
    const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(qrs, qrow[qb] * D + 32 * g + 16, 0, 0);
    qf8[qb] = cat8(lo, hi);
  }

  f32x4 acc_o[NQB][NDB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int j = 0; j < NDB; ++j) acc_o[qb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float os[NQB] = {0.f, 0.f};  // final factor s_v,ref / l per query

  if constexpr (SPARSE) {
    if (a.N < 0) { Ks[tid] = 0; Vs[tid] = 0; }  // see the bf16 kernel
    const int beg = a.row_ptr[(size_t)bh * a.T + qa];
    const int end = a.row_ptr[(size_t)bh * a.T + qa + 1];
    // tile indices and their K and V scales, 64 at a time, one per lane
    int colv = beg + lane < end ? a.col_idx[beg + lane] : -1;
    float svv = (colv >= 0 && colv < a.T) ? SV[colv] : 0.f;
    float skv = (colv >= 0 && colv < a.T) ? SK[colv] : 0.f;
    float svref = svv;
    for (int j = beg + 64; j < end; ++j) {  // rows longer than 64 entries
      const int c = a.col_idx[j];
      if (c >= 0 && c < a.T) svref = fmaxf(svref, SV[c]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) svref = fmaxf(svref, __shfl_xor(svref, o, 64));
    svref = uniform_f(svref);
    const float c0 = sq * a.scale_log2;
    // per entry of the index block (one per lane): valid keys, exp2 multiplier,
    // log2 and inverse of s_v / s_v,ref; the steps read them with readlane
    int kvv;
    float ckv, lrv, irv;
    auto derive = [&]() {
      const bool ok = colv >= 0 && colv < a.T;
      kvv = ok ? min(64, a.N - colv * 64) : 0;
      ckv = ok ? c0 * skv : 1.f;  // a missing tile's scores are all -inf: any positive multiplier
      lrv = ok ? __log2f(svv / svref) : 0.f;  // P' = P * s_v / s_v,ref
      irv = ok ? svref / svv : 0.f;
    };
    derive();
    float m[NQB] = {-INFINITY, -INFINITY};
    f32x4 acc_l[NQB];  // rows 0 and 1 (lane group 0): sums of P' over tile 0 and tile 1 of each pair
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) acc_l[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float lsum[NQB] = {0.f, 0.f};
    // exact sums of the unrounded P, kept only for the log-sum-exp output
    const bool want_lse = a.lse != nullptr;
    float lex[NQB] = {0.f, 0.f};
    // ones operand for those sums: row 0 holds 1.0 on tile-0 keys, row 1 on tile-1 keys
    const uint32_t one4 = 0x38383838u;  // four E4M3 codes of 1.0
    const i32x8_t onesf = (l16 == 0) ? i32x8_t{(int)one4, (int)one4, (int)one4, (int)one4, 0, 0, 0, 0}
                        : (l16 == 1) ? i32x8_t{0, 0, 0, 0, (int)one4, (int)one4, (int)one4, (int)one4}
                                     : i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    // wave w loads tile w of each pair: its K tile and its V^T tile (8 KB each)
    static_assert(NI * 1024 == KT && KT == VT, "one tile per wave");
    int koff[NI], voff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int lin = 1024 * i + 16 * lane;
      const int rk = lin / D, pk = (lin % D) / 16;
      koff[i] = rk * D + 16 * (pk ^ swz_k8(rk));
      const int rv = lin / 64, pv = (lin % 64) / 16;
      voff[i] = rv * 64 + 16 * (pv ^ swz_v8(rv));
    }
    // col0, col1: the pair's tile indices (-1 for none); out-of-range columns load zeros
    auto issue_k = [&](int col0, int col1) {
      const int cb = (w ? col1 : col0) * KT;
      static_for<0, NI>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        lds_dma16<1024 * i>(krs, Ks + KT * w, cb + koff[i]);
      });
    };
    auto issue_v = [&](int col0, int col1) {
      const int cb = (w ? col1 : col0) * VT;
      static_for<0, NI>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        lds_dma16<1024 * i>(vrs, Vs + VT * w, cb + voff[i]);
      });
    };
    auto col_at = [&](int j) { return j < end ? __builtin_amdgcn_readlane(colv, (j - beg) & 63) : -1; };
    // fragment read addresses: K row 16 (kb % 4) + l16 of tile kb / 4, granules 2g and 2g + 1;
    // V^T row 16 jd + l16 of each tile, granule g
    const int fk = swz_k8(l16);
    const int ka0 = l16 * D + 16 * ((2 * g) ^ fk), ka1 = l16 * D + 16 * ((2 * g + 1) ^ fk);
    const int va = l16 * 64 + 16 * (g ^ swz_v8(l16));
    int c0i = col_at(beg), c1i = col_at(beg + 1);
    if (beg < end) {
      issue_k(c0i, c1i);
      issue_v(c0i, c1i);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(NI));  // this wave's K share has landed
      lds_barrier();
    }
    for (int j = beg; j < end; j += 2) {
      const bool more = j + 2 < end;
      int kv[2];
      float ck[2], lr[2], ir[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {  // a pair never straddles a block of 64 indices
        const int e = (j + t - beg) & 63;
        kv[t] = __builtin_amdgcn_readlane(kvv, e);
        ck[t] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ckv), e));
        lr[t] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lrv), e));
        ir[t] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(irv), e));
      }
      if (((j - beg) & 63) == 62 && more) {  // the next pair starts a new block of 64 indices
        // (only rows longer than 64 entries get here; waits for the loads in flight)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        colv = j + 2 + lane < end ? a.col_idx[j + 2 + lane] : -1;
        svv = (colv >= 0 && colv < a.T) ? SV[colv] : 0.f;
        skv = (colv >= 0 && colv < a.T) ? SK[colv] : 0.f;
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        derive();
      }
      const int n0 = more ? col_at(j + 2) : -1, n1 = more ? col_at(j + 3) : -1;
      const bool work = kv[0] + kv[1] > 0;
      i32x8_t pf[NQB];
      if (work) {
        // S^T = K Q^T over both tiles: key blocks 0..3 from tile 0, 4..7 from tile 1
        f32x4 s[NQB][8];
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
          const uint8_t* kp = Ks + (kb >> 2) * KT + 16 * (kb & 3) * D;
          const i32x8_t kf = cat8(*reinterpret_cast<const u32x4*>(kp + ka0), *reinterpret_cast<const u32x4*>(kp + ka1));
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) s[qb][kb] = mma_fp8(kf, qf8[qb], f32x4{0.f, 0.f, 0.f, 0.f});
        }
        if (__builtin_expect(kv[0] < 64 || kv[1] < 64, 0)) {  // keys past N or of a missing tile do not exist
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
            for (int kb = 0; kb < 8; ++kb)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (16 * (kb & 3) + 4 * g + i >= kv[kb >> 2]) s[qb][kb][i] = -INFINITY;
        }
        // row max in log2 units from each tile's raw max (the multipliers are positive)
        bool raise = false;
        float mloc[NQB];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          float mt[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const float mx = smax(smax(smax4(s[qb][4 * t]), smax4(s[qb][4 * t + 1])),
                                  smax(smax4(s[qb][4 * t + 2]), smax4(s[qb][4 * t + 3])));
            mt[t] = kv[t] > 0 ? mx * ck[t] : -INFINITY;
          }
          mloc[qb] = smax(mt[0], mt[1]);
          raise |= mloc[qb] > m[qb] + 8.f;
        }
        if (__ballot(raise)) {
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) {
            const float mtt = group4_max(mloc[qb]);
            const float mn = mtt > m[qb] + 8.f ? fmaxf(m[qb], mtt) : m[qb];
            const float alpha = __builtin_amdgcn_exp2f(m[qb] - mn);
            m[qb] = mn;
#pragma unroll
            for (int jd = 0; jd < NDB; ++jd) acc_o[qb][jd] *= alpha;
            lsum[qb] *= alpha;
            lex[qb] *= alpha;
          }
        }
        // P' -> fp8, B operand of the PV step: byte 4 kb + i of lane group g is
        // key 16 (kb % 4) + 4g + i of tile kb / 4
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const float b0 = lr[0] - m[qb], b1 = lr[1] - m[qb];
#pragma unroll
          for (int kb = 0; kb < 8; ++kb) {
            const float mul = kb < 4 ? ck[0] : ck[1], add = kb < 4 ? b0 : b1;
#pragma unroll
            for (int i = 0; i < 4; ++i) s[qb][kb][i] = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][i], mul, add));
          }
          if (__builtin_expect(want_lse, 0)) {  // one branch for the step, not one per key block
            float part[2] = {0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) part[kb >> 2] += (s[qb][kb][0] + s[qb][kb][1]) + (s[qb][kb][2] + s[qb][kb][3]);
            lex[qb] += part[0] * ir[0] + part[1] * ir[1];  // per-lane partial sums of P'; ir undoes the V-scale ratio
          }
#pragma unroll
          for (int kb = 0; kb < 8; ++kb) {
            // the low half first, the high half second: the word passed as the
            // first step's untouched high half is overwritten, so it may be any
            // register (the first input's own bits: no zero to materialise)
            int wd = __builtin_amdgcn_cvt_pk_fp8_f32(s[qb][kb][0], s[qb][kb][1], __float_as_int(s[qb][kb][0]), false);
            wd = __builtin_amdgcn_cvt_pk_fp8_f32(s[qb][kb][2], s[qb][kb][3], wd, true);
            pf[qb][kb] = wd;
          }
          const f32x4 r = mma_fp8(onesf, pf[qb], f32x4{0.f, 0.f, 0.f, 0.f});
          lsum[qb] += r[0] * ir[0] + r[1] * ir[1];  // meaningful in lane group 0
        }
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // this wave's V share has landed
      lds_barrier();                              // V visible; both waves are done with K
      if (more) issue_k(n0, n1);                  // the next K pair loads during the PV step
      if (work) {
        // O^T += V^T P'^T: lane (d row, g) reads 16 codes of each tile
#pragma unroll
        for (int jd = 0; jd < NDB; ++jd) {
          const uint8_t* vp = Vs + 16 * jd * 64 + va;
          const i32x8_t vf = cat8(*reinterpret_cast<const u32x4*>(vp), *reinterpret_cast<const u32x4*>(vp + VT));
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) acc_o[qb][jd] = mma_fp8(vf, pf[qb], acc_o[qb][jd]);
        }
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // this wave's share of the next K pair has landed
      lds_barrier();                              // next K visible; both waves are done with V
      if (more) issue_v(n0, n1);
      c0i = n0;
      c1i = n1;
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const float lt = __shfl(lsum[qb], l16, 64);  // from lane group 0
      os[qb] = lt > 0.f ? svref / lt : 0.f;
      const float le = group4_sum(lex[qb]);
      if (want_lse && g == 0 && qvalid[qb])
        a.lse[(size_t)bh * a.N_pad + qrow[qb]] = le > 0.f ? (m[qb] + __log2f(le)) * kLn2 : -INFINITY;
    }
  }

  f32x4 acc_n[NQB][NDB];
  float inv_den[NQB] = {0.f, 0.f};
  if constexpr (LINEAR) {
    // the readout runs on bf16 operands holding the exact code values
    Frag<bf16_t> qfb[NQB][D / 32];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const uint2 u = *reinterpret_cast<const uint2*>(
            Q + (size_t)(qvalid[qb] ? qrow[qb] : 0) * D + 32 * c + 8 * g);
        codes_to_bf16(qfb[qb][c], qvalid[qb] ? u.x : 0u, qvalid[qb] ? u.y : 0u);
      }
    readout<bf16_t, D, R, NQB>(readout_src<bf16_t, D, R>(a, bh), qfb, qrow, qvalid, lane, acc_n, inv_den, sq);
  }
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    bf16_t* O = reinterpret_cast<bf16_t*>(a.o) + base + (size_t)qrow[qb] * D;
#pragma unroll
    for (int jd = 0; jd < NDB; ++jd) {
      float r4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = 0.f;
        if constexpr (SPARSE) x += acc_o[qb][jd][i] * os[qb];
        if constexpr (LINEAR) x += acc_n[qb][jd][i] * inv_den[qb];
        r4[i] = qvalid[qb] ? x : 0.f;
      }
      st4o(O + 16 * jd + 4 * g, r4[0], r4[1], r4[2], r4[3]);
    }
  }
}

template <int R>
static hipError_t attend_dispatch_fp8(const AttendArgs& a, bool sparse, bool linear, hipStream_t st) {
  const long grid = 8 * (a.nrows / a.T) * ((a.T + 7) / 8);
  if (sparse && linear) k_attend_fp8<R, true, true><<<grid, 128, 0, st>>>(a);
  else if (sparse) k_attend_fp8<R, true, false><<<grid, 128, 0, st>>>(a);
  else k_attend_fp8<R, false, true><<<grid, 128, 0, st>>>(a);
  return hipGetLastError();
}

static inline hipError_t attend_fp8_by_shape(const Shape& s, const AttendArgs& a, bool sparse, bool linear,
                                             hipStream_t st) {
  if (!linear || s.rank == 16) return attend_dispatch_fp8<16>(a, sparse, linear, st);
  if (s.rank == 32) return attend_dispatch_fp8<32>(a, sparse, linear, st);
  return attend_dispatch_fp8<64>(a, sparse, linear, st);
}

// Launch helpers shared by the bf16/fp8 translation unit and the float32 one.
template <typename T, int D, int R>
static hipError_t attend_dispatch(const AttendArgs& a, bool sparse, bool linear, hipStream_t st) {
  const long grid = 8 * (a.nrows / a.T) * ((a.T + 7) / 8);
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
