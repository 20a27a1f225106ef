// Linear branch over the complement of the kept tiles.  For the queries of
// tile a the sums S and z of the rotary low-rank branch run over the valid
// keys outside the kept tiles M_a only: the context the block-sparse branch
// leaves out (SparkDiffusion news article, section 05: the linear branch
// restores what the sparsification discards; SLA in the 2026-05-02 survey post
// on sparse attention for video generation routes the non-critical weights to
// linear attention).
//
// The streaming pass writes every key tile's own state S_b = sum_{j in b}
// k'_j v_j^T (parameter type) and feature sum z_b; the finalize step writes
// the full S (float) and W_o^T.  Both states are stored in the order of the
// readout's A fragments of S^T, so sums taken element by element are
// fragments already.  One block per
// (b, h, query tile a), 4 waves of 16 queries:
//  1. flags of the tiles in CSR row a (entries outside [0, T) and repeats
//     name no extra tile); a row keeping every tile has no complement keys
//     and leaves O as it is;
//  2. S_c = S - sum_{b in M_a} S_b and z_c = z - sum z_b, or, when the row
//     keeps more than half of the tiles, S_c = sum_{b not in M_a} S_b (so that
//     a small complement is never the difference of two large sums); float
//     sums in ascending tile order, every thread owning fixed 8-element
//     fragment slots, four tiles' loads in flight;
//  3. S_c as readout A fragments in LDS (bf16 hi + lo halves, or float);
//  4. per wave: phi_q = elu(q U_q) + 1, q' = rope(phi_q), n = q' S_c,
//     den = phi_q . z_c, then O_lW^T = W_o^T (n / den)^T on the matrix cores
//     (n split into bf16 hi + lo halves), added to the O_s already in o (the
//     hybrid) or written with zero pad rows (the branch alone).
#pragma once

#include "common.hpp"
#include "kernels.hpp"
#include "readout.hpp"

namespace hsa {

// Query tiles per block of the complement kernel.
#ifndef HSA_COMPL_ROWS
#define HSA_COMPL_ROWS 4
#endif
constexpr int kComplRows = HSA_COMPL_ROWS;

struct ComplArgs {
  int N, N_pad, T, H;
  int gt, gh, gw;
  const void* q;           // [BH][N_pad][d] storage type
  const float* qs;         // fp8: [BH][T] Q tile scales
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const void* tile_s;      // [BH][T][NFE] parameter type, readout fragment order
  const float* tile_z;     // [BH][T][r]
  const float* s_full;     // [BH][NFE] float, readout fragment order
  const float* z;          // [BH][r]
  const void* uq_frag;     // [H] U_q^T A fragments
  const void* wo_frag;     // [H] W_o^T A fragments
  const float2* rope;
  void* o;                 // [BH][N_pad][d] output type
  int add;                 // 1: add O_lW to the O_s held in o; 0: write O_lW (pad rows 0)
  long nrows;
};

// 8 consecutive state elements of the parameter type (one fragment slot
// group), loaded as one unit: 16 bytes of bf16 or 32 bytes of float.
template <typename OT, int CE> struct StateChunk;
template <> struct StateChunk<bf16_t, 8> {
  u32x4 w;
  __device__ void load(const bf16_t* p) { w = *reinterpret_cast<const u32x4*>(p); }
  __device__ float get(int s) const { return bf16_bits_to_f32((w[s >> 1] >> (16 * (s & 1))) & 0xFFFFu); }
};
template <> struct StateChunk<float, 8> {
  float4 a, b;
  __device__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ float get(int s) const {
    const float4& v = s < 4 ? a : b;
    switch (s & 3) { case 0: return v.x; case 1: return v.y; case 2: return v.z; default: return v.w; }
  }
};
// Output element access: 4 consecutive values of a row of o.
__device__ __forceinline__ void add4_out(bf16_t* p, const f32x4& x) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  const float a0 = bf16_bits_to_f32(u.x & 0xFFFFu) + x[0], a1 = bf16_bits_to_f32(u.x >> 16) + x[1];
  const float a2 = bf16_bits_to_f32(u.y & 0xFFFFu) + x[2], a3 = bf16_bits_to_f32(u.y >> 16) + x[3];
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a0, a1), pack_bf16x2(a2, a3));
}
__device__ __forceinline__ void add4_out(float* p, const f32x4& x) {
  float4 u = *reinterpret_cast<const float4*>(p);
  u.x += x[0]; u.y += x[1]; u.z += x[2]; u.w += x[3];
  *reinterpret_cast<float4*>(p) = u;
}
__device__ __forceinline__ void put4_out(bf16_t* p, const f32x4& x) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
}
__device__ __forceinline__ void put4_out(float* p, const f32x4& x) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}

// T: storage type of Q (float, bf16_t or fp8_t); OT: parameter / operand type
// (float for float inputs, bf16_t otherwise); output type = OT.  G: query
// tiles per block.  Neighbouring query tiles keep many of the same key tiles
// (at 720P four consecutive rows name about half as many distinct tiles as
// they hold entries), so a block gathers the union of its rows' tiles once and
// adds each state to the rows that take it.
template <typename T, typename OT, int D, int R, int G>
__global__ __launch_bounds__(256, 2) void k_compl(ComplArgs a) {
  constexpr int NDB = D / 16, NRB = R / 16, NRC = (R + 31) / 32;
  constexpr int NFE = NDB * NRC * 512;            // elements of one set of state fragments
  constexpr bool SPLIT = sizeof(OT) == 2;         // bf16 operands: hi + lo halves
  constexpr int CE = 8;                           // one fragment slot group per load
  constexpr int NCH = NFE / (256 * CE);           // slot groups per thread
  constexpr int U = SPLIT ? 4 : 2;                // tiles in flight
  constexpr int SFB = (SPLIT ? 2 : 1) * NFE * (int)sizeof(OT);
  constexpr int LISTB = (G + 4) * kComplMaxT;     // G flag bytes per tile + 4-byte list entries
  static_assert(NCH >= 1 && NFE % (256 * CE) == 0, "state split");
  static_assert(G >= 1 && G <= 8, "rows per block");
  __shared__ __align__(16) uint8_t lds[SFB > LISTB ? SFB : LISTB];
  // bf16 operands: the head's W_o^T fragments staged once per block (32 KB at
  // d = 128), read by every row's output step from LDS instead of L2 (float
  // operands would need twice that and read them from memory)
  constexpr int NWE = NDB * (D / 32) * 512;
  __shared__ __align__(16) OT WOs[SPLIT ? NWE : 8];
  __shared__ float ZC[R];
  __shared__ int wcnt[4];
  __shared__ int nkept_sh[G];

  const int TG = (a.T + G - 1) / G;  // row groups per (b, h)
  const int L = uniform(head_interleaved_row(blockIdx.x, TG));
  if (L < 0) return;
  const int bh = uniform(L / TG), a0 = uniform((L - bh * TG) * G);
  const int ng = min(G, a.T - a0);
  const int h = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  if constexpr (SPLIT) {  // published by the first barrier below
    const OT* wsrc = reinterpret_cast<const OT*>(a.wo_frag) + (size_t)h * NWE;
    for (int e = 8 * tid; e < NWE; e += 8 * 256)
      *reinterpret_cast<u32x4*>(&WOs[e]) = *reinterpret_cast<const u32x4*>(wsrc + e);
  }
  uint8_t* kept = lds;                                                       // [G][kComplMaxT]
  uint32_t* list = reinterpret_cast<uint32_t*>(lds + G * kComplMaxT);        // tile | row mask << 16

  // ---- 1. each row's tile flags and their count
  for (int r = 0; r < G; ++r)
    for (int b = tid; b < a.T; b += 256) kept[r * kComplMaxT + b] = 0;
  if (tid < G) nkept_sh[tid] = 0;
  __syncthreads();
  for (int r = 0; r < ng; ++r) {
    const int beg = a.row_ptr[(size_t)bh * a.T + a0 + r], end = a.row_ptr[(size_t)bh * a.T + a0 + r + 1];
    for (int j = beg + tid; j < end; j += 256) {
      const int b = a.col_idx[j];
      if (b >= 0 && b < a.T) kept[r * kComplMaxT + b] = 1;
    }
  }
  __syncthreads();
  for (int r = 0; r < ng; ++r) {
    int mine = 0;
    for (int b = tid; b < a.T; b += 256) mine += kept[r * kComplMaxT + b];
    if (mine) atomicAdd(&nkept_sh[r], mine);
  }
  __syncthreads();
  // per row: 0 no key outside the kept tiles (O_l = 0); 1 subtract the kept
  // tiles' states from S; 2 sum the other tiles' states
  int mode[G];
#pragma unroll
  for (int r = 0; r < G; ++r) {
    const int nk = r < ng ? uniform(nkept_sh[r]) : a.T;
    mode[r] = nk >= a.T ? 0 : (2 * nk <= a.T ? 1 : 2);
  }

  // ---- 2. ascending list of the tiles any row takes, then the float sums
  int cnt = 0;
  for (int cb = 0; cb < a.T; cb += 256) {
    const int b = cb + tid;
    uint32_t m = 0;
    if (b < a.T) {
#pragma unroll
      for (int r = 0; r < G; ++r) {
        const bool k = kept[r * kComplMaxT + b] != 0;
        if ((mode[r] == 1 && k) || (mode[r] == 2 && !k)) m |= 1u << r;
      }
    }
    const bool f = m != 0;
    const uint64_t bal = __ballot(f);
    if (lane == 0) wcnt[w] = __popcll(bal);
    __syncthreads();
    int off = cnt;
    for (int i = 0; i < w; ++i) off += wcnt[i];
    if (f) {
      const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
      list[off + rank] = (uint32_t)b | (m << 16);
    }
    cnt += wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
    __syncthreads();
  }
  cnt = uniform(cnt);

  const size_t sbase = (size_t)bh * NFE;
  const OT* TS = reinterpret_cast<const OT*>(a.tile_s) + (size_t)bh * a.T * NFE;
  const float* TZ = a.tile_z + (size_t)bh * a.T * R;
  float acc[G][NCH][CE];
  float zc[G];
  {
    float sf[NCH][CE];
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
      for (int s = 0; s < CE; ++s) sf[i][s] = a.s_full[sbase + CE * (tid + 256 * i) + s];
    const float zf = tid < R ? a.z[(size_t)bh * R + tid] : 0.f;
#pragma unroll
    for (int r = 0; r < G; ++r) {
#pragma unroll
      for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int s = 0; s < CE; ++s) acc[r][i][s] = mode[r] == 1 ? sf[i][s] : 0.f;
      zc[r] = mode[r] == 1 ? zf : 0.f;
    }
  }
  for (int j0 = 0; j0 < cnt; j0 += U) {
    StateChunk<OT, CE> x[U][NCH];
    float zx[U];
    uint32_t msk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = j0 + u < cnt;
      const uint32_t e = ok ? (uint32_t)uniform((int)list[j0 + u]) : 0u;
      const int b = (int)(e & 0xFFFFu);
      msk[u] = e >> 16;
      const OT* src = TS + (size_t)b * NFE;
#pragma unroll
      for (int i = 0; i < NCH; ++i) x[u][i].load(src + CE * (tid + 256 * i));
      zx[u] = (tid < R) ? TZ[(size_t)b * R + tid] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int r = 0; r < G; ++r) {
        if (msk[u] & (1u << r)) {
          const float sg = mode[r] == 1 ? -1.f : 1.f;
#pragma unroll
          for (int i = 0; i < NCH; ++i)
#pragma unroll
            for (int s = 0; s < CE; ++s) acc[r][i][s] = fmaf(sg, x[u][i].get(s), acc[r][i][s]);
          zc[r] = fmaf(sg, zx[u], zc[r]);
        }
      }
    }
  }

  // ---- 3, 4. per row: S_c as readout A fragments, then the readout of its
  // 64 queries (16 per wave), W_o, added to O_s or written
  OT* SF = reinterpret_cast<OT*>(lds);
  const size_t base = (size_t)bh * a.N_pad * D;
  const OT* UQ = reinterpret_cast<const OT*>(a.uq_frag) + (size_t)h * NRB * (D / 32) * 512;
  const OT* WO = reinterpret_cast<const OT*>(a.wo_frag) + (size_t)h * NDB * (D / 32) * 512;
#pragma unroll
  for (int r = 0; r < G; ++r) {
    if (r >= ng) break;
    const int qa = a0 + r;
    const int qrow = qa * 64 + 16 * w + l16;
    const bool qvalid = qrow < a.N;
    OT* O = reinterpret_cast<OT*>(a.o) + base + (size_t)qrow * D;
    if (mode[r] == 0) {
      if (!a.add) {
#pragma unroll
        for (int jo = 0; jo < NDB; ++jo) put4_out(O + 16 * jo + 4 * g, f32x4{0.f, 0.f, 0.f, 0.f});
      }
      continue;
    }
    __syncthreads();  // the flags and list, or the previous row's fragments, are no longer read
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int e = CE * (tid + 256 * i);
      const float* x = acc[r][i];
      if constexpr (SPLIT) {
        u32x4 hi, lo;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float h0 = bf16_bits_to_f32(f32_to_bf16_bits(x[2 * p]));
          const float h1 = bf16_bits_to_f32(f32_to_bf16_bits(x[2 * p + 1]));
          hi[p] = pack_bf16x2(h0, h1);
          lo[p] = pack_bf16x2(x[2 * p] - h0, x[2 * p + 1] - h1);
        }
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(SF) + e) = hi;
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(SF) + NFE + e) = lo;
      } else {
        float* dst = reinterpret_cast<float*>(SF) + e;
        reinterpret_cast<float4*>(dst)[0] = make_float4(x[0], x[1], x[2], x[3]);
        reinterpret_cast<float4*>(dst)[1] = make_float4(x[4], x[5], x[6], x[7]);
      }
    }
    if (tid < R) ZC[tid] = zc[r];
    __syncthreads();

    Frag<OT> qf[D / 32];
    float qscale = 1.f;
    if constexpr (sizeof(T) == 1) {
      const uint8_t* Q = reinterpret_cast<const uint8_t*>(a.q) + base;
      qscale = a.qs[(size_t)bh * a.T + qa];
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const uint2 u = qvalid ? *reinterpret_cast<const uint2*>(Q + (size_t)qrow * D + 32 * c + 8 * g)
                               : make_uint2(0, 0);
        codes_to_bf16(qf[c], u.x, u.y);
      }
    } else {
      const OT* Q = reinterpret_cast<const OT*>(a.q) + base;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        if (qvalid) load8(qf[c], Q + (size_t)qrow * D + 32 * c + 8 * g);
        else qf[c].zero();
      }
    }
    ReadoutSrc<OT> src;
    src.uq = UQ;
    src.sp = SF;
    src.z = ZC;
    src.rope = a.rope;
    src.gt = a.gt; src.gh = a.gh; src.gw = a.gw;
    f32x4 acc_n[1][NDB];
    float inv_den[1];
    readout<OT, D, R, 1>(src, &qf, &qrow, &qvalid, lane, acc_n, inv_den, qscale);

    // n / den as B fragments of a contraction over d: slot s of lane group g
    // in chunk c is dim 16 (2c + s/4) + 4g + s%4 (W_o^T fragments use the same order)
    Frag<OT> nh[D / 32], nl[D / 32];
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      float x[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) x[s] = acc_n[0][2 * c + (s >> 2)][s & 3] * inv_den[0];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        if constexpr (SPLIT) {
          const float h0 = bf16_bits_to_f32(f32_to_bf16_bits(x[2 * p]));
          const float h1 = bf16_bits_to_f32(f32_to_bf16_bits(x[2 * p + 1]));
          nh[c].set_pair(p, h0, h1);
          nl[c].set_pair(p, x[2 * p] - h0, x[2 * p + 1] - h1);
        } else {
          nh[c].set_pair(p, x[2 * p], x[2 * p + 1]);
        }
      }
    }
#pragma unroll
    for (int jo = 0; jo < NDB; ++jo) {
      f32x4 acc_w = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        Frag<OT> wf;
        if constexpr (SPLIT) wf.w = *reinterpret_cast<const u32x4*>(&WOs[((jo * (D / 32) + c) * 64 + lane) * 8]);
        else load8(wf, WO + ((size_t)(jo * (D / 32) + c) * 64 + lane) * 8);
        mma(acc_w, wf, nh[c]);
        if constexpr (SPLIT) mma(acc_w, wf, nl[c]);
      }
      if (a.add) {
        if (qvalid) add4_out(O + 16 * jo + 4 * g, acc_w);
      } else {
        put4_out(O + 16 * jo + 4 * g, qvalid ? acc_w : f32x4{0.f, 0.f, 0.f, 0.f});
      }
    }
  }
}

template <typename T, typename OT, int D, int R>
static hipError_t compl_dispatch(const ComplArgs& a, hipStream_t st) {
  constexpr int G = kComplRows;
  const int tg = (a.T + G - 1) / G;
  const long grid = 8 * (a.nrows / a.T) * ((tg + 7) / 8);
  k_compl<T, OT, D, R, G><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <typename T, typename OT>
static hipError_t compl_by_shape(const Shape& s, const ComplArgs& a, hipStream_t st) {
  if (s.d == 64) {
    if (s.rank == 16) return compl_dispatch<T, OT, 64, 16>(a, st);
    if (s.rank == 32) return compl_dispatch<T, OT, 64, 32>(a, st);
    return compl_dispatch<T, OT, 64, 64>(a, st);
  }
  if (s.rank == 16) return compl_dispatch<T, OT, 128, 16>(a, st);
  if (s.rank == 32) return compl_dispatch<T, OT, 128, 32>(a, st);
  return compl_dispatch<T, OT, 128, 64>(a, st);
}

hipError_t launch_compl_f32(const Shape& s, const ComplArgs& a, hipStream_t st);

}  // namespace hsa
