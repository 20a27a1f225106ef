// Backward pass of the hybrid attention on a fixed mask: dQ, dK, dV (float32)
// for an upstream dO, through both branches.  The forward is the RoLA hybrid
// of the SparkDiffusion news article, section 05 (block-sparse softmax branch
// + rotary low-rank linear branch); the gradients are those of that function
// with the tile selection held fixed (it is piecewise constant in the inputs).
//
// Sparse branch (softmax recomputed from the forward's log-sum-exp, as flash
// attention does):  P = exp(scale q k^T - lse), dP = dO v^T,
//   dS = P * (dP - D) with D_i = dO_i . O_s,i,
//   dq = scale dS k,  dk = scale dS^T q,  dv = P^T dO.
// The dQ kernels walk each query tile's CSR row, the dK/dV kernels each key
// tile's column of the transposed mask (CSC, built by k_csc_*).  For bf16
// inputs the tiles are staged by LDS-direct loads into XOR-swizzled LDS
// tiles, once for row reads and once for transposing reads (ds_read_b64_tr_b16
// gives the transposed operands), with 32 rows per wave.
//
// Linear branch, O_l = num / den, num = rho(phi(q U_q)) S, den = phi(q U_q) . z:
//   gW = dO W_o^T, dnum = gW / den, dden = -(gW . O_l) / den,
//   dq' = S dnum,  dS = sum_i q'_i dnum_i^T,  dz = sum_i dden_i phi_q,i,
//   dq = ((dden z + rho^T dq') * phi'(x_q)) U_q^T,
//   dk' = dS v,  dv = dS^T k',  dk = ((dz + rho^T dk') * phi'(x_k)) U_k^T.
// k_bwd_q makes the query-side pass (dq of the linear branch, D, and partial
// dS, dz per block), k_bwd_fin sums the partials in a fixed order, k_bwd_k
// makes the key-side pass (dk, dv of the linear branch).  The sparse kernels
// then add their parts.
//
// Matrix-core operands follow the fragment convention of common.hpp.  Where an
// accumulator (lane: column l % 16, rows 4 (l / 16) + i) feeds a contraction
// over its rows, two 16-row blocks form one 32-wide chunk, slot s of lane
// group g holding row 16 (s / 4) + 4 g + s % 4; the other operand is read in
// the same order (LDS tiles staged with that permutation, or two 4-element
// runs from memory).
#pragma once

#include "common.hpp"
#include "kernels.hpp"
#include "lds_dma.hpp"
#include "readout.hpp"

namespace hsa {

struct BwdArgs {
  int N, N_pad, T, H, nchunk, tpc;
  int tpc_k;  // key tiles per block of the key-side linear pass
  int gt, gh, gw;
  float scale;             // softmax scale
  const void* q;
  const void* k;
  const void* v;
  const void* dout;        // dO, [BH][N_pad][d] in the input type
  const void* uq;          // [H][d][r] parameter type
  const void* uk;
  const void* wo;          // [H][d][d]
  const int32_t* row_ptr;  // the forward's mask (CSR)
  const int32_t* col_idx;
  const int32_t* col_ptr;  // its transpose (CSC): query tiles per key tile, ascending
  const int32_t* row_idx;
  long csc_cap;            // entries row_idx holds
  const int32_t* col_order; // [BH*T] key tiles in the order the dK / dV blocks take them
  const void* os;          // [BH][N_pad][d] O_s in the output type
  const float* lse;        // [BH][N_pad] natural-log log-sum-exp of the sparse branch
  float* dsum;             // [BH][N_pad] D_i
  const float* z;          // [BH][R]
  const float* s_frag;     // [BH][NFE] S^T as float readout A fragments
  const float* s_pfrag;    // [BH][R*D] S in perm_frag_index order
  const void* wob_frag;    // [H][D*D] W_o as A fragments
  const void* uqp_frag;    // [H] U_q in perm_frag_index order
  void* ukp_frag;          // [H] U_k in perm_frag_index order (written by k_bwd_fin)
  const void* uq_frag;     // [H] U_q^T A fragments
  void* uk_frag;           // [H] U_k^T A fragments (written by k_bwd_fin)
  const float2* rope;
  float* part_ds;          // [BH][nchunk][R][D]
  float* part_dz;          // [BH][nchunk][R]
  float* ds_plain;         // [BH][R][D]
  float* ds_frag;          // [BH][NFE] dS^T as float A fragments
  float* dz;               // [BH][R]
  float* dq;               // [BH][N_pad][D] float
  float* dk;
  float* dv;
  long nrows;
};

// ------------------------------------------------------------ small helpers
// 8 floats -> operand fragment(s): bf16 hi + lo halves (x = hi + lo to ~2^-17),
// or the floats themselves.
__device__ __forceinline__ void split8(const float* x, Frag<bf16_t>& hi, Frag<bf16_t>& lo) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float h0 = bf16_bits_to_f32(f32_to_bf16_bits(x[2 * p]));
    const float h1 = bf16_bits_to_f32(f32_to_bf16_bits(x[2 * p + 1]));
    hi.set_pair(p, h0, h1);
    lo.set_pair(p, x[2 * p] - h0, x[2 * p + 1] - h1);
  }
}
__device__ __forceinline__ void split8(const float* x, Frag<float>& hi, Frag<float>& lo) {
#pragma unroll
  for (int s = 0; s < 8; ++s) hi.v[s] = x[s];
  lo.zero();
}
// acc += (hi + lo) b; float operands need no low half.
template <typename OT>
__device__ __forceinline__ void mma_hl(f32x4& acc, const Frag<OT>& hi, const Frag<OT>& lo, const Frag<OT>& b) {
  mma(acc, hi, b);
  if constexpr (sizeof(OT) == 2) mma(acc, lo, b);
}
// B fragment of a contraction over accumulator rows: blocks lo (rows 0..15)
// and hi (rows 16..31) of one 32-wide chunk, each value times m.
template <typename OT>
__device__ __forceinline__ void pack_rows(Frag<OT>& f, const f32x4& lo, const f32x4& hi, float m) {
  f.set_pair(0, lo[0] * m, lo[1] * m);
  f.set_pair(1, lo[2] * m, lo[3] * m);
  f.set_pair(2, hi[0] * m, hi[1] * m);
  f.set_pair(3, hi[2] * m, hi[3] * m);
}
__device__ __forceinline__ void load8f(float* x, const float* p) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
// 8 elements of the storage type (or of float) as floats
__device__ __forceinline__ void load8_any(float* x, const bf16_t* p) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int s = 0; s < 8; ++s) x[s] = bf16_bits_to_f32((w[s >> 1] >> (16 * (s & 1))) & 0xFFFFu);
}
__device__ __forceinline__ void load8_any(float* x, const float* p) { load8f(x, p); }
// Fragment loads from a per-head parameter array through one buffer
// descriptor: the lane's byte offset in a register and the fragment's offset
// as a scalar, so that a loop over many fragments holds no address register
// per fragment (64-bit per-fragment addresses, hoisted out of the tile loop,
// would not fit beside the loop's values).
__device__ __forceinline__ void fload(Frag<bf16_t>& f, __amdgpu_buffer_rsrc_t r, int voff, int soff) {
  f.w = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ void fload(Frag<float>& f, __amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff + 16, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) { f.v[i] = __uint_as_float(a[i]); f.v[4 + i] = __uint_as_float(b[i]); }
}
__device__ __forceinline__ void fload8f(float* x, __amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff + 16, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) { x[i] = __uint_as_float(a[i]); x[4 + i] = __uint_as_float(b[i]); }
}
// (cos, sin) of the rotation of feature pair jp (0 .. r/2 - 1) at latent
// position (t, y, x)
template <int R>
__device__ __forceinline__ float2 rope_at(const float2* rope, int gt, int gh, int t, int y, int x, int jp) {
  constexpr int ht = 3 * R / 16, hh = 3 * R / 16, hwp = R / 8;
  if (jp < ht) return rope[t * ht + jp];
  if (jp < ht + hh) return rope[gt * ht + y * hh + (jp - ht)];
  return rope[gt * ht + gh * hh + x * hwp + (jp - ht - hh)];
}

// ------------------------------------------------- staging for the sparse kernels
// Swizzle of a staged tile read both ways: by 16-byte row reads over 16
// consecutive rows (operand fragments) and by transposing 8-byte reads over
// aligned groups of 8 rows, each row giving one 32-byte granule pair.  With
// rr the row's 256-byte bank-set index (RG 16-byte granules per row),
// granule g sits at g ^ f(rr), f = 2 (rr mod RG/2) + (rr div RG/2) mod 2:
// over 16 rows f takes every value, so a row read hits 16 distinct granule
// positions, and over each group of 8 rows f / 2 takes distinct values, so a
// transposing read hits distinct granule pairs.
template <int RG> __device__ __forceinline__ int swz_kt(int row) {
  const int rr = row / (16 / RG);
  return 2 * (rr & (RG / 2 - 1)) + ((rr / (RG / 2)) & 1);
}
// dma_offsets with that swizzle (NW waves share the tile's loads).
template <int RB, int NW = 2>
__device__ __forceinline__ void dma_offsets_kt(int w, int lane, int* off) {
  constexpr int RG = RB / 16, NI = 64 * RB / 1024 / NW;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int lin = 1024 * (NI * w + i) + 16 * lane;
    const int row = lin / RB, pos = (lin % RB) / 16;
    off[i] = row * RB + 16 * (pos ^ swz_kt<RG>(row));
  }
}
// One 4-byte-per-lane LDS-direct load (lane l writes 4 bytes at lds_dst +
// 4 l), issued like lds_dma16 and counted by the kernel's own vmcnt waits.
__device__ __forceinline__ void lds_dma4(const i32x4_t& rs, const void* lds_dst, int voff) {
  const uint32_t m0v = (uint32_t)(uintptr_t)(lds_void_t)(lds_dst);
  uint32_t keep;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %1, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
               : "=&s"(keep) : "v"(voff), "s"(m0v), "s"(rs) : "memory");
}

// ------------------------------------------------- transposed mask (CSC)
static __global__ void k_zero_i32(int n, int32_t* __restrict__ p) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// The transposed mask through a bit matrix per (b, h): bit (b, a) is set when
// row a keeps tile b (repeated entries set it once).  Counting and listing the
// set bits of each column in index order gives the CSC rows ascending, with
// no sort and independent of the order the bits were set in.
// one thread per CSR row (b, h, a)
static __global__ __launch_bounds__(256) void k_csc_bits(int rows, int T, int W, const int32_t* __restrict__ row_ptr,
                                                          const int32_t* __restrict__ col_idx, uint32_t* __restrict__ bits) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  const int bh = r / T, a = r - bh * T;
  for (int j = row_ptr[r]; j < row_ptr[r + 1]; ++j) {
    const int b = col_idx[j];
    if (b >= 0 && b < T) atomicOr(&bits[((size_t)bh * T + b) * W + (a >> 5)], 1u << (a & 31));
  }
}

// one thread per column (b, h, tile): LIST = false counts its bits, true lists them
template <bool LIST>
__global__ __launch_bounds__(256) void k_csc_cols(int cols, int W, const uint32_t* __restrict__ bits,
                                                  int32_t* __restrict__ cnt, const int32_t* __restrict__ col_ptr,
                                                  int32_t* __restrict__ row_idx, long cap) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= cols) return;
  const uint32_t* row = bits + (size_t)c * W;
  if constexpr (!LIST) {
    int n = 0;
    for (int i = 0; i < W; ++i) n += __popc(row[i]);
    cnt[c] = n;
  } else {
    long pos = col_ptr[c];
    for (int i = 0; i < W; ++i) {
      uint32_t m = row[i];
      while (m) {
        const int bit = __ffs(m) - 1;
        m &= m - 1;
        if (pos < cap) row_idx[pos] = 32 * i + bit;
        ++pos;
      }
    }
  }
}

static __global__ __launch_bounds__(1024) void k_csc_scan(int n, const int32_t* __restrict__ cnt,
                                                          int32_t* __restrict__ ptr) {
  __shared__ int32_t part[1024];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < n; base += 1024) {
    const int i = base + threadIdx.x;
    const int v = i < n ? cnt[i] : 0;
    part[threadIdx.x] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int t = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
      __syncthreads();
      part[threadIdx.x] += t;
      __syncthreads();
    }
    if (i < n) ptr[i] = carry + part[threadIdx.x] - v;
    __syncthreads();
    if (threadIdx.x == 1023) carry += part[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) ptr[n] = carry;
}

// Order in which the dK / dV kernels take the key tiles of each head.  The
// tiles are sorted by column length (the query tiles that keep the tile) in
// buckets of 2^kOrderShift lengths, longest first, then by tile index: column
// lengths run from 0 to several times the mean, and in index order a long
// column that starts late decides when the launch ends.  The sorted list is
// then dealt to the XCDs (block p runs on XCD p mod 8) in runs of kOrderRun
// consecutive entries, snaking, so that each XCD's L2 sees runs of
// neighbouring key tiles, which share many of their query tiles, while every
// XCD still draws from the whole list.  No result depends on the order (each column is
// handled by one block wherever it stands).  One block per (b, h): a bitonic
// sort of (bucket << 16 | tile) keys in LDS, for T <= kOrderMaxT.
constexpr int kOrderShift = 6;
constexpr int kOrderRun = 16;
constexpr int kOrderMaxT = 2048;
static __global__ __launch_bounds__(1024) void k_csc_order(int T, const int32_t* __restrict__ col_ptr, long cap,
                                                           int32_t* __restrict__ order) {
  __shared__ uint32_t key[kOrderMaxT];
  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * T;
  for (int i = tid; i < kOrderMaxT; i += 1024) {
    uint32_t k = 0xFFFFFFFFu;  // past T: sorts last
    if (i < T) {
      const long b = min((long)col_ptr[c0 + i], cap), e = min((long)col_ptr[c0 + i + 1], cap);
      const int len = (int)max(0L, min(e - b, (long)T));
      k = ((uint32_t)(T - len) >> kOrderShift) << 16 | (uint32_t)i;
    }
    key[i] = k;
  }
  __syncthreads();
  for (int k = 2; k <= kOrderMaxT; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < kOrderMaxT; i += 1024) {
        const int l = i ^ j;
        if (l > i) {
          const uint32_t x = key[i], y = key[l];
          if ((x > y) == ((i & k) == 0)) {
            key[i] = y;
            key[l] = x;
          }
        }
      }
      __syncthreads();
    }
  // dispatch position p -> sorted position: within each group of 8 kOrderRun
  // entries, XCD x takes run x, the XCDs in reverse order every other group
  // (so that no XCD always takes the longest run of a group); the last
  // partial group stays in place
  constexpr int G = 8 * kOrderRun;
  const int full = T / G * G;
  for (int p = tid; p < T; p += 1024) {
    int q = p;
    if (p < full) {
      const int x = p & 7, j = p >> 3, grp = j / kOrderRun;
      q = G * grp + kOrderRun * ((grp & 1) ? 7 - x : x) + j % kOrderRun;
    }
    order[c0 + p] = c0 + (int)(key[q] & 0xFFFFu);
  }
}
// Plain order (head-major), where T is too large for the sort's LDS.
static __global__ void k_iota_i32(int n, int32_t* __restrict__ p) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = i;
}

// --------------------------------------------------------- sparse: dQ
// float32 inputs: one block per query tile (4 waves x 16 queries), over its
// CSR row; K, V and K^T (keys permuted for the dS contraction) staged in LDS
// through registers, the next tile prefetched into registers.  Adds
// scale * dS K to dq.  (bf16 inputs use k_bwd_dq_bf16 below.)
template <typename T, int D>
__global__ __launch_bounds__(256) void k_bwd_dq(BwdArgs a) {
  constexpr int CPR = D / 8, NVU = 16 * CPR;   // threads staging 4 keys x 8 dims each
  constexpr int KSTR = D + 8, VSTR = 64 + 8, NDB = D / 16;
  __shared__ __align__(16) T Ks[64 * KSTR];
  __shared__ __align__(16) T Vs[64 * KSTR];
  __shared__ __align__(16) T Kt[D * VSTR];

  const int L = uniform(head_interleaved_row(blockIdx.x, a.T));
  if (L < 0) return;
  const int bh = uniform(L / a.T), qa = uniform(L - bh * a.T);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const size_t base = (size_t)bh * a.N_pad * D;
  const T* Q = reinterpret_cast<const T*>(a.q) + base;
  const T* K = reinterpret_cast<const T*>(a.k) + base;
  const T* V = reinterpret_cast<const T*>(a.v) + base;
  const T* G = reinterpret_cast<const T*>(a.dout) + base;
  const int qrow = qa * 64 + 16 * w + l16;
  const bool qvalid = qrow < a.N;
  Frag<T> qf[D / 32], gf[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    if (qvalid) {
      load8(qf[c], Q + (size_t)qrow * D + 32 * c + 8 * g);
      load8(gf[c], G + (size_t)qrow * D + 32 * c + 8 * g);
    } else {
      qf[c].zero();
      gf[c].zero();
    }
  }
  const float c2 = a.scale * kLog2e;
  const float lse2 = qvalid ? a.lse[(size_t)bh * a.N_pad + qrow] * kLog2e : 0.f;
  const float dd = qvalid ? a.dsum[(size_t)bh * a.N_pad + qrow] : 0.f;
  f32x4 acc[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int beg = a.row_ptr[(size_t)bh * a.T + qa], end = a.row_ptr[(size_t)bh * a.T + qa + 1];
  const int kg = tid % 16, c8 = tid / 16;
  Chunk8<T> kc[4], vc[4];
  auto load_tile = [&](int col) {
    const bool ok = col >= 0 && col < a.T;
    if (tid < NVU) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int gr = col * 64 + 4 * kg + ii;
        if (ok && gr < a.N) {
          gload8(kc[ii], K + (size_t)gr * D + c8 * 8);
          gload8(vc[ii], V + (size_t)gr * D + c8 * 8);
        } else {
          zero8(kc[ii]);
          zero8(vc[ii]);
        }
      }
    }
  };
  if (beg < end) load_tile(a.col_idx[beg]);
  for (int j = beg; j < end; ++j) {
    const int col = a.col_idx[j];
    __syncthreads();  // the previous tile's LDS reads are done
    if (tid < NVU) {
      const int p0 = vt_pos_a(4 * kg);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        lds_row(&Ks[(4 * kg + ii) * KSTR + c8 * 8], kc[ii]);
        lds_row(&Vs[(4 * kg + ii) * KSTR + c8 * 8], vc[ii]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        st4v(&Kt[(c8 * 8 + e) * VSTR + p0], elem(kc[0], e), elem(kc[1], e), elem(kc[2], e), elem(kc[3], e));
    }
    __syncthreads();
    if (j + 1 < end) load_tile(a.col_idx[j + 1]);
    const int kvalid = (col >= 0 && col < a.T) ? min(64, a.N - col * 64) : 0;
    if (kvalid <= 0) continue;
    f32x4 s[4], dp[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      dp[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        Frag<T> kf, vf;
        load8(kf, &Ks[(16 * kb + l16) * KSTR + 32 * c + 8 * g]);
        load8(vf, &Vs[(16 * kb + l16) * KSTR + 32 * c + 8 * g]);
        mma(s[kb], kf, qf[c]);
        mma(dp[kb], vf, gf[c]);
      }
    }
    // dS^T (keys x queries), scale folded in
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = (16 * kb + 4 * g + i < kvalid) ? exp2f(fmaf(s[kb][i], c2, -lse2)) : 0.f;
        s[kb][i] = p * (dp[kb][i] - dd) * a.scale;
      }
    Frag<T> dsf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) pack_rows(dsf[c], s[2 * c], s[2 * c + 1], 1.f);
#pragma unroll
    for (int jd = 0; jd < NDB; ++jd)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        Frag<T> ktf;
        load8(ktf, &Kt[(16 * jd + l16) * VSTR + 32 * c + 8 * g]);
        mma(acc[jd], ktf, dsf[c]);
      }
  }
  if (qvalid) {
    float* out = a.dq + base + (size_t)qrow * D;
#pragma unroll
    for (int jd = 0; jd < NDB; ++jd) {
      float4 o = *reinterpret_cast<float4*>(out + 16 * jd + 4 * g);
      o.x += acc[jd][0]; o.y += acc[jd][1]; o.z += acc[jd][2]; o.w += acc[jd][3];
      *reinterpret_cast<float4*>(out + 16 * jd + 4 * g) = o;
    }
  }
}

// bf16 sparse dQ: one block per query tile = NW waves of 64 / NW queries
// (4 x 16: 162 registers, three waves per SIMD within the 48 KB of LDS a
// block stages; 2 x 32 would let each fragment read from LDS feed two
// matrix-core steps, but at 256 registers and 48 KB only three blocks fit a
// CU, one and a half waves per SIMD).  K and V
// tiles go global -> LDS by LDS-direct loads into XOR-swizzled tiles; the K
// tile, double-buffered, is read both by rows (S = Q K^T) and transposed
// (dq += scale dS K), so each key tile is staged once.  The next K tile loads
// during the scores step, the next V tile during the dq step.
template <int D, int NW>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 3 : 2) void k_bwd_dq_bf16(BwdArgs a) {
  constexpr int RB = 2 * D, RG = RB / 16;
  constexpr int NQB = 2 * 2 / NW, NDB = D / 16;  // 16-query blocks per wave
  constexpr int NI = 64 * RB / 1024 / NW;   // LDS-direct loads per wave per tile
  __shared__ __align__(16) uint8_t Kb[2][64 * RB];
  __shared__ __align__(16) uint8_t Vs[64 * RB];

  const int L = uniform(head_interleaved_row(blockIdx.x, a.T));
  if (L < 0) return;
  const int bh = uniform(L / a.T), qa = uniform(L - bh * a.T);
  const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const size_t base = (size_t)bh * a.N_pad * D;
  const bf16_t* Q = reinterpret_cast<const bf16_t*>(a.q) + base;
  const bf16_t* G = reinterpret_cast<const bf16_t*>(a.dout) + base;
  const int nbytes = a.N * RB;
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc((void*)Q, 0, nbytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t grs = __builtin_amdgcn_make_buffer_rsrc((void*)G, 0, nbytes, kBufferFlags);
  const i32x4_t krs = make_rsrc_regs(reinterpret_cast<const bf16_t*>(a.k) + base, nbytes);
  const i32x4_t vrs = make_rsrc_regs(reinterpret_cast<const bf16_t*>(a.v) + base, nbytes);

  int qrow[NQB];
  bool qvalid[NQB];
  float lse2[NQB], dd[NQB];
  Frag<bf16_t> qf[NQB][D / 32], gf[NQB][D / 32];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    qrow[qb] = qa * 64 + 16 * NQB * w + 16 * qb + l16;
    qvalid[qb] = qrow[qb] < a.N;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {  // rows >= N read as zeros
      qf[qb][c].w = __builtin_amdgcn_raw_buffer_load_b128(qrs, (qrow[qb] * D + 32 * c + 8 * g) * 2, 0, 0);
      gf[qb][c].w = __builtin_amdgcn_raw_buffer_load_b128(grs, (qrow[qb] * D + 32 * c + 8 * g) * 2, 0, 0);
    }
    lse2[qb] = qvalid[qb] ? a.lse[(size_t)bh * a.N_pad + qrow[qb]] * kLog2e : 0.f;
    dd[qb] = qvalid[qb] ? a.dsum[(size_t)bh * a.N_pad + qrow[qb]] : 0.f;
  }
  f32x4 acc[NQB][NDB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int j = 0; j < NDB; ++j) acc[qb][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (a.N < 0) { Kb[0][tid] = 0; Kb[1][tid] = 0; Vs[tid] = 0; }  // (the tiles are written by LDS-direct loads only)
  const int beg = a.row_ptr[(size_t)bh * a.T + qa], end = a.row_ptr[(size_t)bh * a.T + qa + 1];
  const float c2 = a.scale * kLog2e;
  int koff[NI], voff[NI];
  dma_offsets_kt<RB, NW>(w, lane, koff);
  dma_offsets<RB, false, NW>(w, lane, voff);
  const int kaddr = l16 * RB + 16 * (g ^ swz_kt<RG>(l16));
  const int vaddr = l16 * RB + 16 * (g ^ swz_k<RG>(l16));
  const int rowl = 4 * g + (l16 >> 2);
  const int taddr = rowl * RB + 16 * (((l16 >> 1) & 1) ^ swz_kt<RG>(rowl)) + 8 * (l16 & 1);
  int colv = beg + lane < end ? a.col_idx[beg + lane] : 0;
  int col = __builtin_amdgcn_readlane(colv, 0);
  int ncol = __builtin_amdgcn_readlane(colv, 1);
  if (beg < end) {
    dma_tile<RB, NW>(krs, col, koff, Kb[0], w);
    dma_tile<RB, NW>(vrs, col, voff, Vs, w);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
  }
  for (int j = beg; j < end; ++j) {
    const int cur = (j - beg) & 1;
    const bool more = j + 1 < end;
    if (more) dma_tile<RB, NW>(krs, ncol, koff, Kb[cur ^ 1], w);  // that buffer was last read by the previous dq step
    const uint8_t* Kc = Kb[cur];
    const int kvalid = (col >= 0 && col < a.T) ? min(64, a.N - col * 64) : 0;
    Frag<bf16_t> dsf[NQB][2];
    if (kvalid > 0) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {  // key blocks 2c, 2c + 1 -> chunk c of dS^T
        f32x4 s[NQB][2], dp[NQB][2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int kb = 2 * c + h2;
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) {
            s[qb][h2] = f32x4{0.f, 0.f, 0.f, 0.f};
            dp[qb][h2] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int cc = 0; cc < D / 32; ++cc) {
            Frag<bf16_t> kf, vf;
            kf.w = *reinterpret_cast<const u32x4*>(&Kc[(kaddr ^ (64 * cc)) + 16 * RB * kb]);
            vf.w = *reinterpret_cast<const u32x4*>(&Vs[(vaddr ^ (64 * cc)) + 16 * RB * kb]);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
              mma(s[qb][h2], kf, qf[qb][cc]);
              mma(dp[qb][h2], vf, gf[qb][cc]);
            }
          }
        }
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          if (D == 128 && kvalid == 64) {  // keys past N exist only in the ragged last tile (d = 64 keeps one
                                            // form: the second would cost it a wave per SIMD)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                s[qb][h2][i] = __builtin_amdgcn_exp2f(fmaf(s[qb][h2][i], c2, -lse2[qb])) * (dp[qb][h2][i] - dd[qb]) * a.scale;
          } else {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int key = 16 * (2 * c + h2) + 4 * g + i;
                const float p = key < kvalid ? __builtin_amdgcn_exp2f(fmaf(s[qb][h2][i], c2, -lse2[qb])) : 0.f;
                s[qb][h2][i] = p * (dp[qb][h2][i] - dd[qb]) * a.scale;
              }
          }
          pack_rows(dsf[qb][c], s[qb][0], s[qb][1], 1.f);
        }
      }
    }
    lds_barrier();  // both waves are done with V
    if (more) dma_tile<RB, NW>(vrs, ncol, voff, Vs, w);
    if (kvalid > 0) {
#pragma unroll
      for (int jd = 0; jd < NDB; ++jd) {
        const int ta = taddr ^ (32 * jd);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          Frag<bf16_t> ktf;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const s16x4_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(&Kc[ta + (32 * c + 16 * hh) * RB]));
            const uint2 u = __builtin_bit_cast(uint2, t);
            ktf.w[2 * hh] = u.x;
            ktf.w[2 * hh + 1] = u.y;
          }
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) mma(acc[qb][jd], ktf, dsf[qb][c]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // this wave's shares of the next K and V have landed
    lds_barrier();                              // next K, V visible; both waves are done with this K
    if (((j + 2 - beg) & 63) == 0 && j + 2 < end) {
      colv = j + 2 + lane < end ? a.col_idx[j + 2 + lane] : 0;
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    col = ncol;
    ncol = __builtin_amdgcn_readlane(colv, (j + 2 - beg) & 63);
  }
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    if (!qvalid[qb]) continue;
    float* out = a.dq + base + (size_t)qrow[qb] * D;
#pragma unroll
    for (int jd = 0; jd < NDB; ++jd) {
      float4 o = *reinterpret_cast<float4*>(out + 16 * jd + 4 * g);
      o.x += acc[qb][jd][0]; o.y += acc[qb][jd][1]; o.z += acc[qb][jd][2]; o.w += acc[qb][jd][3];
      *reinterpret_cast<float4*>(out + 16 * jd + 4 * g) = o;
    }
  }
}

// ------------------------------------------------------- sparse: dK, dV
// float32 inputs: one block per key tile (4 waves x 16 keys), over the query
// tiles that keep it (CSC, ascending); Q, dO, their transposes (queries
// permuted) and the per-query lse and D staged in LDS.  Adds scale * dS^T Q
// to dk and P^T dO to dv.  (bf16 inputs use k_bwd_dkv_bf16 below.)
template <typename T, int D>
__global__ __launch_bounds__(256) void k_bwd_dkv(BwdArgs a) {
  constexpr int CPR = D / 8, NVU = 16 * CPR;
  constexpr int KSTR = D + 8, VSTR = 64 + 8, NDB = D / 16;
  __shared__ __align__(16) T Qs[64 * KSTR];
  __shared__ __align__(16) T Gs[64 * KSTR];
  __shared__ __align__(16) T Qt[D * VSTR];
  __shared__ __align__(16) T Gt[D * VSTR];
  __shared__ float ls[64];
  __shared__ float dsm[64];

  const int L = uniform(head_interleaved_row(blockIdx.x, a.T));
  if (L < 0) return;
  const int bh = uniform(L / a.T), kt = uniform(L - bh * a.T);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const size_t base = (size_t)bh * a.N_pad * D;
  const T* Q = reinterpret_cast<const T*>(a.q) + base;
  const T* K = reinterpret_cast<const T*>(a.k) + base;
  const T* V = reinterpret_cast<const T*>(a.v) + base;
  const T* G = reinterpret_cast<const T*>(a.dout) + base;
  const int krow = kt * 64 + 16 * w + l16;
  const bool kvalid = krow < a.N;
  Frag<T> kf[D / 32], vf[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    if (kvalid) {
      load8(kf[c], K + (size_t)krow * D + 32 * c + 8 * g);
      load8(vf[c], V + (size_t)krow * D + 32 * c + 8 * g);
    } else {
      kf[c].zero();
      vf[c].zero();
    }
  }
  const float c2 = a.scale * kLog2e;
  f32x4 acck[NDB], accv[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j) {
    acck[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    accv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int beg = a.col_ptr[(size_t)bh * a.T + kt];
  const int end = (int)min((long)a.col_ptr[(size_t)bh * a.T + kt + 1], a.csc_cap);
  const int kg = tid % 16, c8 = tid / 16;
  Chunk8<T> qc[4], gc[4];
  float lsv = INFINITY, dv0 = 0.f;
  auto load_tile = [&](int row) {
    if (tid < NVU) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int gr = row * 64 + 4 * kg + ii;
        if (gr < a.N) {
          gload8(qc[ii], Q + (size_t)gr * D + c8 * 8);
          gload8(gc[ii], G + (size_t)gr * D + c8 * 8);
        } else {
          zero8(qc[ii]);
          zero8(gc[ii]);
        }
      }
    }
    if (tid < 64) {
      const int gr = row * 64 + tid;
      lsv = gr < a.N ? a.lse[(size_t)bh * a.N_pad + gr] * kLog2e : INFINITY;  // no such query: P = 0
      dv0 = gr < a.N ? a.dsum[(size_t)bh * a.N_pad + gr] : 0.f;
    }
  };
  if (beg < end) load_tile(a.row_idx[beg]);
  for (int j = beg; j < end; ++j) {
    __syncthreads();
    if (tid < NVU) {
      const int p0 = vt_pos_a(4 * kg);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        lds_row(&Qs[(4 * kg + ii) * KSTR + c8 * 8], qc[ii]);
        lds_row(&Gs[(4 * kg + ii) * KSTR + c8 * 8], gc[ii]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        st4v(&Qt[(c8 * 8 + e) * VSTR + p0], elem(qc[0], e), elem(qc[1], e), elem(qc[2], e), elem(qc[3], e));
        st4v(&Gt[(c8 * 8 + e) * VSTR + p0], elem(gc[0], e), elem(gc[1], e), elem(gc[2], e), elem(gc[3], e));
      }
    }
    if (tid < 64) {
      ls[tid] = lsv;
      dsm[tid] = dv0;
    }
    __syncthreads();
    if (j + 1 < end) load_tile(a.row_idx[j + 1]);
    // S, dP: queries x this wave's 16 keys; lane: key column, query rows 16 qb + 4 g + i
    f32x4 s[4], dp[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      s[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
      dp[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        Frag<T> qfr, gfr;
        load8(qfr, &Qs[(16 * qb + l16) * KSTR + 32 * c + 8 * g]);
        load8(gfr, &Gs[(16 * qb + l16) * KSTR + 32 * c + 8 * g]);
        mma(s[qb], qfr, kf[c]);
        mma(dp[qb], gfr, vf[c]);
      }
    }
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ql = 16 * qb + 4 * g + i;
        const float p = exp2f(fmaf(s[qb][i], c2, -ls[ql]));
        s[qb][i] = p;
        dp[qb][i] = p * (dp[qb][i] - dsm[ql]) * a.scale;
      }
    Frag<T> pf[2], dsf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      pack_rows(pf[c], s[2 * c], s[2 * c + 1], 1.f);
      pack_rows(dsf[c], dp[2 * c], dp[2 * c + 1], 1.f);
    }
#pragma unroll
    for (int jd = 0; jd < NDB; ++jd)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        Frag<T> gtf, qtf;
        load8(gtf, &Gt[(16 * jd + l16) * VSTR + 32 * c + 8 * g]);
        load8(qtf, &Qt[(16 * jd + l16) * VSTR + 32 * c + 8 * g]);
        mma(accv[jd], gtf, pf[c]);
        mma(acck[jd], qtf, dsf[c]);
      }
  }
  if (kvalid) {
    float* ok = a.dk + base + (size_t)krow * D;
    float* ov = a.dv + base + (size_t)krow * D;
#pragma unroll
    for (int jd = 0; jd < NDB; ++jd) {
      float4 x = *reinterpret_cast<float4*>(ok + 16 * jd + 4 * g);
      x.x += acck[jd][0]; x.y += acck[jd][1]; x.z += acck[jd][2]; x.w += acck[jd][3];
      *reinterpret_cast<float4*>(ok + 16 * jd + 4 * g) = x;
      float4 y = *reinterpret_cast<float4*>(ov + 16 * jd + 4 * g);
      y.x += accv[jd][0]; y.y += accv[jd][1]; y.z += accv[jd][2]; y.w += accv[jd][3];
      *reinterpret_cast<float4*>(ov + 16 * jd + 4 * g) = y;
    }
  }
}

// ---------------------------------------------------- linear: query side
// One block per (b, h, pair of chunks of query tiles) = two groups of 4 waves
// x 16 queries per tile, one group per chunk.  Per query: the readout's
// forward quantities (x_q, phi_q, q', num, den), gW, D = dO . O_s, the linear
// branch's dq (written to dq: the sparse kernel adds to it), and the
// contributions to dS (through LDS: dnum and q' of the 64 queries, contracted
// over queries on the matrix cores) and dz.  One partial dS, dz per chunk.
template <typename T, int D, int R>
__global__ __launch_bounds__(512, 1) void k_bwd_q(BwdArgs a) {
  constexpr int NDB = D / 16, NRB = R / 16, NRC = (R + 31) / 32;
  constexpr int NFE = NDB * NRC * 512;
  constexpr int GST = D + 4, QST = R + 4;       // LDS row strides (floats)
  constexpr int NB = NDB * NRB, NBW = NB / 4;    // 16x16 blocks of dS^T, per wave
  static_assert(NB % 4 == 0, "dS blocks per wave");
  // bf16 operands: q' of the tile's queries is kept in LDS as the bf16 values
  // the dS product packs it to (float operands keep floats), and the head's
  // W_o^T fragments (32 KB at d = 128) are staged once per block, so that the
  // gW step reads them from LDS instead of from L2 for every tile and wave
  constexpr bool BF = sizeof(T) == 2;
  constexpr int QSTB = R + 8;                    // bf16 q' row stride (elements)
  constexpr int NUF = NRB * (D / 32) * 512, NUP = NDB * NRC * 512;  // elements of the U_q operands
  // per group: dnum and q' of the group's tile; shared: W_o^T, U_q^T and U_q fragments
  __shared__ __align__(16) float GNa[2][64 * GST];
  __shared__ __align__(16) float QPa[2][BF ? 4 : 64 * QST];
  __shared__ __align__(16) uint16_t QPBa[2][BF ? 64 * QSTB : 8];
  __shared__ __align__(16) T WOS[BF ? D * D : 8];
  __shared__ __align__(16) T UQFS[BF ? NUF : 8];
  __shared__ __align__(16) T UQPS[BF ? NUP : 8];
  __shared__ float zred[2][4][R];

  // XCD-aware order: the hardware hands block i to XCD i % 8; all chunks of
  // (b, h) run on XCD bh % 8, so each XCD's L2 holds the per-head operand
  // fragments (~128 KB) of a few heads only.
  // Two groups of 4 waves per block: group grp takes chunk 2 c + grp of the
  // (b, h)'s query tiles, exactly the tiles (and order) a chunk's own block
  // would take, and writes that chunk's partial sums; the groups share the
  // head's operand fragments staged in LDS.
  const int npair = (a.nchunk + 1) / 2;
  const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
  const int bh = xcd + 8 * (jx / npair), cpair = jx % npair;
  if (bh >= (int)(a.nrows / a.T)) return;
  const int h = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, grp = tid >> 8, w = (tid >> 6) & 3;
  const int chunk = 2 * cpair + grp;
  const int t0 = chunk * a.tpc, t1 = min(a.T, t0 + a.tpc);  // empty for a chunk past the last
  const int niter = min(a.T - 2 * cpair * a.tpc, a.tpc);     // the first chunk of the pair is the longer
  float* GN = GNa[grp];
  float* QP = QPa[grp];
  uint16_t* QPB = QPBa[grp];
  const int l16 = lane & 15, g = lane >> 4;
  const size_t base = (size_t)bh * a.N_pad * D;
  const T* Q = reinterpret_cast<const T*>(a.q) + base;
  const T* G = reinterpret_cast<const T*>(a.dout) + base;
  const T* OS = reinterpret_cast<const T*>(a.os) + base;
  const T* UQF = reinterpret_cast<const T*>(a.uq_frag) + (size_t)h * NRB * (D / 32) * 512;
  // parameter operands in fragment order: every fragment load reads one contiguous run
  const T* UQP = reinterpret_cast<const T*>(a.uqp_frag) + (size_t)h * NDB * NRC * 512;
  const T* WOB = reinterpret_cast<const T*>(a.wob_frag) + (size_t)h * D * D;
  const float* SF = a.s_frag + (size_t)bh * NFE;
  const float* SPF = a.s_pfrag + (size_t)bh * R * D;
  const float* Z = a.z + (size_t)bh * R;
  // the parameter fragments through buffer descriptors (see fload)
  constexpr int FB = 64 * 8 * (int)sizeof(T);  // bytes of one operand fragment
  const __amdgpu_buffer_rsrc_t r_uqf = make_rsrc(UQF, NRB * (D / 32) * FB);
  const __amdgpu_buffer_rsrc_t r_uqp = make_rsrc(UQP, NDB * NRC * FB);
  const __amdgpu_buffer_rsrc_t r_wob = make_rsrc(WOB, D * D * (int)sizeof(T));
  const __amdgpu_buffer_rsrc_t r_sf = make_rsrc(SF, NFE * 4);
  const __amdgpu_buffer_rsrc_t r_spf = make_rsrc(SPF, R * D * 4);
  const int lo_t = lane * 8 * (int)sizeof(T), lo_f = lane * 32;  // the lane's byte offsets in a fragment
  if constexpr (BF) {
    for (int i = tid; i < D * D / 8; i += 512)
      reinterpret_cast<u32x4*>(WOS)[i] = reinterpret_cast<const u32x4*>(WOB)[i];
    for (int i = tid; i < NUF / 8; i += 512)
      reinterpret_cast<u32x4*>(UQFS)[i] = reinterpret_cast<const u32x4*>(UQF)[i];
    for (int i = tid; i < NUP / 8; i += 512)
      reinterpret_cast<u32x4*>(UQPS)[i] = reinterpret_cast<const u32x4*>(UQP)[i];
    __syncthreads();
  }

  f32x4 dsacc[NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i) dsacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dzl[NRB][4];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) dzl[rb][i] = 0.f;

  for (int it = 0; it < niter; ++it) {  // the same count in both groups (the barriers pair up)
    const int t = t0 + it;
    const bool live = t < t1;
    if (live) {
    const int qrow = t * 64 + 16 * w + l16;
    const bool qvalid = qrow < a.N;
    Frag<T> qf[D / 32], gf[D / 32];
    float gos = 0.f;  // dO . O_s, this lane's share
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      if (qvalid) {
        load8(qf[c], Q + (size_t)qrow * D + 32 * c + 8 * g);
        load8(gf[c], G + (size_t)qrow * D + 32 * c + 8 * g);
        float gx[8], ox[8];
        load8_any(gx, G + (size_t)qrow * D + 32 * c + 8 * g);
        load8_any(ox, OS + (size_t)qrow * D + 32 * c + 8 * g);
#pragma unroll
        for (int e = 0; e < 8; ++e) gos = fmaf(gx[e], ox[e], gos);
      } else {
        qf[c].zero();
        gf[c].zero();
      }
    }
    gos = group4_sum(gos);
    // x_q^T = U_q^T q^T; phi; den; q' = rope(phi) (x_q itself is not kept: phi'(x) is 1 where
    // phi > 1 and phi elsewhere)
    const int ql = 16 * w + l16;
    const int tok = qvalid ? qrow : 0;
    int pt, py, px;  // the query's latent position
    {
      const int hw = a.gh * a.gw, rem = tok - (tok / hw) * hw;
      pt = tok / hw;
      py = rem / a.gw;
      px = rem - py * a.gw;
    }
    float fq[NRB][4];
    float den = 0.f;
    Frag<T> qpf[NRC];
    {
      float qp[NRB][4];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        f32x4 xq = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          Frag<T> uf;
          if constexpr (BF) load8(uf, UQFS + ((rb * (D / 32) + c) * 64 + lane) * 8);
          else fload(uf, r_uqf, lo_t, (rb * (D / 32) + c) * FB);
          mma(xq, uf, qf[c]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          fq[rb][i] = elu1(xq[i]);
          den = fmaf(fq[rb][i], Z[16 * rb + 4 * g + i], den);
        }
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const float2 cs = rope_at<R>(a.rope, a.gt, a.gh, pt, py, px, (16 * rb + 4 * g) / 2 + pr);
          const float x0 = fq[rb][2 * pr], x1 = fq[rb][2 * pr + 1];
          qp[rb][2 * pr] = x0 * cs.x - x1 * cs.y;
          qp[rb][2 * pr + 1] = x0 * cs.y + x1 * cs.x;
        }
        // q' of the tile's queries for the dS product (the previous tile's product is done)
        if constexpr (BF)
          *reinterpret_cast<uint2*>(&QPB[ql * QSTB + 16 * rb + 4 * g]) =
              make_uint2(pack_bf16x2(qp[rb][0], qp[rb][1]), pack_bf16x2(qp[rb][2], qp[rb][3]));
        else
          *reinterpret_cast<float4*>(&QP[ql * QST + 16 * rb + 4 * g]) =
              make_float4(qp[rb][0], qp[rb][1], qp[rb][2], qp[rb][3]);
      }
#pragma unroll
      for (int rc = 0; rc < NRC; ++rc) {
        const f32x4 lo = f32x4{qp[2 * rc][0], qp[2 * rc][1], qp[2 * rc][2], qp[2 * rc][3]};
        const f32x4 hi = (2 * rc + 1 < NRB) ? f32x4{qp[2 * rc + 1][0], qp[2 * rc + 1][1], qp[2 * rc + 1][2],
                                                    qp[2 * rc + 1][3]}
                                            : f32x4{0.f, 0.f, 0.f, 0.f};
        pack_rows(qpf[rc], lo, hi, 1.f);
      }
    }
    den = group4_sum(den);
    const float invden = 1.f / den;
    // gW^T = W_o dO^T, two d blocks at a time: dnum = gW / den as B fragments
    // (chunks of 32 d) and in LDS for the dS product
    Frag<T> gnf[D / 32];
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      f32x4 gw[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int jd = 2 * c + hh;
        gw[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < D / 32; ++cc) {
          Frag<T> wf;
          if constexpr (BF) load8(wf, WOS + ((jd * (D / 32) + cc) * 64 + lane) * 8);
          else fload(wf, r_wob, lo_t, (jd * (D / 32) + cc) * FB);
          mma(gw[hh], wf, gf[cc]);
        }
        *reinterpret_cast<float4*>(&GN[ql * GST + 16 * jd + 4 * g]) =
            make_float4(gw[hh][0] * invden, gw[hh][1] * invden, gw[hh][2] * invden, gw[hh][3] * invden);
      }
      pack_rows(gnf[c], gw[0], gw[1], invden);
    }
    // num^T = S^T q'^T (rows d, query columns); gW . O_l = dnum . num, with this
    // lane's dnum read back from LDS (its own writes)
    float gwol = 0.f;
#pragma unroll
    for (int jd = 0; jd < NDB; ++jd) {
      f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int rc = 0; rc < NRC; ++rc) {
        float x[8];
        fload8f(x, r_sf, lo_f, (jd * NRC + rc) * 64 * 32);
        Frag<T> hi, lo;
        split8(x, hi, lo);
        mma_hl(num, hi, lo, qpf[rc]);
      }
      const float4 gn = *reinterpret_cast<const float4*>(&GN[ql * GST + 16 * jd + 4 * g]);
      gwol = fmaf(gn.x, num[0], gwol);
      gwol = fmaf(gn.y, num[1], gwol);
      gwol = fmaf(gn.z, num[2], gwol);
      gwol = fmaf(gn.w, num[3], gwol);
    }
    gwol = group4_sum(gwol);
    const float gden = -gwol * invden;  // d den = -(gW . O_l) / den
    if (g == 0 && qvalid) a.dsum[(size_t)bh * a.N_pad + qrow] = gos;
    // dq' = S dnum
    f32x4 dqp[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      dqp[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        float x[8];
        fload8f(x, r_spf, lo_f, (rb * (D / 32) + c) * 64 * 32);
        Frag<T> hi, lo;
        split8(x, hi, lo);
        mma_hl(dqp[rb], hi, lo, gnf[c]);
      }
    }
    // dx_q = (dden z + rho^T dq') * phi'(x_q)
    float dx[NRB][4];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const int m = 16 * rb + 4 * g + 2 * pr;
        const float2 cs = rope_at<R>(a.rope, a.gt, a.gh, pt, py, px, m / 2);
        const float x0 = dqp[rb][2 * pr], x1 = dqp[rb][2 * pr + 1];
        const float d0 = fmaf(gden, Z[m], x0 * cs.x + x1 * cs.y);
        const float d1 = fmaf(gden, Z[m + 1], -x0 * cs.y + x1 * cs.x);
        const float f0 = fq[rb][2 * pr], f1 = fq[rb][2 * pr + 1];
        dx[rb][2 * pr] = d0 * (f0 > 1.f ? 1.f : f0);
        dx[rb][2 * pr + 1] = d1 * (f1 > 1.f ? 1.f : f1);
      }
    Frag<T> dxf[NRC];
#pragma unroll
    for (int rc = 0; rc < NRC; ++rc) {
      const f32x4 lo = f32x4{dx[2 * rc][0], dx[2 * rc][1], dx[2 * rc][2], dx[2 * rc][3]};
      const f32x4 hi = (2 * rc + 1 < NRB) ? f32x4{dx[2 * rc + 1][0], dx[2 * rc + 1][1], dx[2 * rc + 1][2],
                                                  dx[2 * rc + 1][3]}
                                          : f32x4{0.f, 0.f, 0.f, 0.f};
      pack_rows(dxf[rc], lo, hi, 1.f);
    }
    float* dqo = a.dq + base + (size_t)qrow * D;
#pragma unroll
    for (int jd = 0; jd < NDB; ++jd) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int rc = 0; rc < NRC; ++rc) {
        Frag<T> uf;
        if constexpr (BF) load8(uf, UQPS + ((jd * NRC + rc) * 64 + lane) * 8);
        else fload(uf, r_uqp, lo_t, (jd * NRC + rc) * FB);
        mma(acc, uf, dxf[rc]);
      }
      *reinterpret_cast<float4*>(dqo + 16 * jd + 4 * g) =
          qvalid ? make_float4(acc[0], acc[1], acc[2], acc[3]) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // contributions to dz
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) dzl[rb][i] = fmaf(gden, fq[rb][i], dzl[rb][i]);
    }
    __syncthreads();
    if (live) {
    // dS^T (d x r) += dnum^T q' over the tile's 64 queries
#pragma unroll
    for (int ii = 0; ii < NBW; ++ii) {
      const int bi = w + 4 * ii, je = bi % NDB, rb = bi / NDB;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float x[8];
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) x[s2] = GN[(32 * c + 8 * g + s2) * GST + 16 * je + l16];
        Frag<T> hi, lo, qb;
        split8(x, hi, lo);
        if constexpr (BF) {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int qq = 32 * c + 8 * g + 2 * p;
            qb.w[p] = (uint32_t)QPB[qq * QSTB + 16 * rb + l16] | ((uint32_t)QPB[(qq + 1) * QSTB + 16 * rb + l16] << 16);
          }
        } else {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int qq = 32 * c + 8 * g + 2 * p;
            qb.set_pair(p, QP[qq * QST + 16 * rb + l16], QP[(qq + 1) * QST + 16 * rb + l16]);
          }
        }
        mma_hl(dsacc[ii], hi, lo, qb);
      }
    }
    }
    __syncthreads();
  }
  // partials: dS [r][d] rows m = 16 rb + l16, columns 16 je + 4 g .. + 3
  const size_t pb = (size_t)bh * a.nchunk + chunk;
  const bool own = t0 < t1;  // this group's chunk exists
#pragma unroll
  for (int ii = 0; ii < (own ? NBW : 0); ++ii) {
    const int bi = w + 4 * ii, je = bi % NDB, rb = bi / NDB;
    *reinterpret_cast<float4*>(&a.part_ds[(pb * R + 16 * rb + l16) * D + 16 * je + 4 * g]) =
        make_float4(dsacc[ii][0], dsacc[ii][1], dsacc[ii][2], dsacc[ii][3]);
  }
  // dz: sum over the 16 query lanes of each lane group, then over the waves
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = dzl[rb][i];
      x += wave_xor(x, 1);
      x += wave_xor(x, 2);
      x += wave_xor(x, 4);
      x += wave_xor(x, 8);
      if (l16 == 0) zred[grp][w][16 * rb + 4 * g + i] = x;
    }
  __syncthreads();
  const int gt_ = tid & 255;
  if (own && gt_ < R)
    a.part_dz[pb * R + gt_] = (zred[grp][0][gt_] + zred[grp][1][gt_]) + (zred[grp][2][gt_] + zred[grp][3][gt_]);
}

// ------------------------------------------------ linear: partial sums
// Per (b, h) and slice of 8 rank rows: dS = sum of the partials (fixed
// order), written plain and as float readout A fragments of dS^T; the first
// slice also writes dz and zero-fills the fragment slots past r, and, for
// the heads of batch 0, U_k^T as A fragments.
template <typename T, int D, int R>
__global__ __launch_bounds__(256) void k_bwd_fin(BwdArgs a) {
  constexpr int NRB = R / 16, NRC = (R + 31) / 32, NFE = (D / 16) * NRC * 512;
  const int tid = threadIdx.x, bh = blockIdx.x, h = bh % a.H;
  const int r0 = blockIdx.y * 8;
  float* fr = a.ds_frag + (size_t)bh * NFE;
  for (int e = tid; e < 8 * D; e += 256) {
    const int rr = r0 + e / D, col = e % D;
    float s = 0.f;
    for (int c = 0; c < a.nchunk; ++c) s += a.part_ds[(((size_t)bh * a.nchunk + c) * R + rr) * D + col];
    a.ds_plain[((size_t)bh * R + rr) * D + col] = s;
    fr[sp_frag_index<D, R>(rr, col)] = s;
  }
  if (blockIdx.y == 0) {
    for (int e = tid; e < (32 * NRC - R) * D; e += 256) fr[sp_frag_index<D, R>(R + e / D, e % D)] = 0.f;
    if (tid < R) {
      float s = 0.f;
      for (int c = 0; c < a.nchunk; ++c) s += a.part_dz[((size_t)bh * a.nchunk + c) * R + tid];
      a.dz[(size_t)bh * R + tid] = s;
    }
    if (bh < a.H) {  // U_k^T fragments: frag (rb, c), lane l, slot s -> U_k[32 c + 8 (l/16) + s][16 rb + l%16]
      const int nue = NRB * (D / 32) * 512;
      const T* U = reinterpret_cast<const T*>(a.uk) + (size_t)h * D * R;
      T* out = reinterpret_cast<T*>(a.uk_frag) + (size_t)h * nue;
      for (int idx = tid; idx < nue; idx += 256) {
        const int s2 = idx & 7, l = (idx >> 3) & 63, f = idx >> 9;
        const int c = f % (D / 32), rbk = f / (D / 32);
        out[idx] = U[(size_t)(32 * c + 8 * (l >> 4) + s2) * R + 16 * rbk + (l & 15)];
      }
      T* pout = reinterpret_cast<T*>(a.ukp_frag) + (size_t)h * (D / 16) * NRC * 512;
      for (int idx = tid; idx < (D / 16) * NRC * 512; idx += 256) {
        int rr, cc;
        perm_frag_source(idx, R, &rr, &cc);
        pout[idx] = cc < R ? U[(size_t)rr * R + cc] : T{};
      }
    }
  }
}

// ------------------------------------------------------ linear: key side
// One block per (b, h, chunk of key tiles) = 8 waves.  The head's operands
// (U_k^T and U_k fragments, dS^T fragments, and dS rows, the latter put in
// fragment order here) are staged in LDS once per block: read per key tile
// from L2 they were six times the tile's own K and V bytes.  Wave pair p
// takes key tiles t0 + p, t0 + p + 4, ..., 2 waves x 32 keys per tile (two
// 16-key column blocks per wave, so every operand fragment read serves both):
// x_k, phi_k, k', then dk' = dS v, dv = dS^T k' and dk = ((dz + rho^T dk') *
// phi'(x_k)) U_k^T, written to dk and dv (pad rows 0; the sparse kernels add
// to them).
template <typename T, int D, int R>
__global__ __launch_bounds__(512, 1) void k_bwd_k(BwdArgs a) {
  constexpr int NDB = D / 16, NRB = R / 16, NRC = (R + 31) / 32;
  constexpr int NFE = NDB * NRC * 512;
  constexpr int NKB = 2;
  constexpr int NUF = NRB * (D / 32) * 512, NUP = NDB * NRC * 512;  // elements of the U_k operands
  __shared__ __align__(16) T UKF[NUF];
  __shared__ __align__(16) T UKP[NUP];
  __shared__ __align__(16) float DSF[NFE];
  __shared__ __align__(16) float DSP[R * D];  // dS rows as A fragments: (rb, c) lane l16 + 16 g -> dS[16 rb + l16][32 c + 8 g ..]
  const int bh = blockIdx.y, h = bh % a.H;
  const int t0 = blockIdx.x * a.tpc_k, t1 = min(a.T, t0 + a.tpc_k);
  if (t0 >= t1) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int pair = w >> 1, wk = w & 1;
  const size_t base = (size_t)bh * a.N_pad * D;
  const T* K = reinterpret_cast<const T*>(a.k) + base;
  const T* V = reinterpret_cast<const T*>(a.v) + base;
  {
    const T* gu = reinterpret_cast<const T*>(a.uk_frag) + (size_t)h * NUF;
    const T* gp = reinterpret_cast<const T*>(a.ukp_frag) + (size_t)h * NUP;
    const float* gs = a.ds_frag + (size_t)bh * NFE;
    const float* gd = a.ds_plain + (size_t)bh * R * D;
    constexpr int EPV = 16 / (int)sizeof(T);  // elements per 16 bytes
    for (int i = tid; i < NUF / EPV; i += 512) reinterpret_cast<u32x4*>(UKF)[i] = reinterpret_cast<const u32x4*>(gu)[i];
    for (int i = tid; i < NUP / EPV; i += 512) reinterpret_cast<u32x4*>(UKP)[i] = reinterpret_cast<const u32x4*>(gp)[i];
    for (int i = tid; i < NFE / 4; i += 512) reinterpret_cast<float4*>(DSF)[i] = reinterpret_cast<const float4*>(gs)[i];
    for (int i = tid; i < R * D / 8; i += 512) {  // 8 consecutive d of one row r: one lane's slots of a fragment
      const int r = i / (D / 8), d0 = 8 * (i % (D / 8));
      const int f = (r / 16) * (D / 32) + d0 / 32, l = (r % 16) + 16 * ((d0 % 32) / 8);
      float4* dst = reinterpret_cast<float4*>(&DSP[(f * 64 + l) * 8]);
      const float4* src = reinterpret_cast<const float4*>(gd + (size_t)r * D + d0);
      dst[0] = src[0];
      dst[1] = src[1];
    }
    __syncthreads();
  }
  const float* DZ = a.dz + (size_t)bh * R;
  for (int kt = t0 + pair; kt < t1; kt += 4) {
    int krow[NKB];
    bool kvalid[NKB];
    Frag<T> kf[NKB][D / 32], vf[NKB][D / 32];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      krow[kb] = kt * 64 + 32 * wk + 16 * kb + l16;
      kvalid[kb] = krow[kb] < a.N;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        if (kvalid[kb]) {
          load8(kf[kb][c], K + (size_t)krow[kb] * D + 32 * c + 8 * g);
          load8(vf[kb][c], V + (size_t)krow[kb] * D + 32 * c + 8 * g);
        } else {
          kf[kb][c].zero();
          vf[kb][c].zero();
        }
      }
    }
    f32x4 xk[NKB][NRB], dkp[NKB][NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        xk[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        dkp[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        Frag<T> uf;
        load8(uf, UKF + ((size_t)(rb * (D / 32) + c) * 64 + lane) * 8);
        float x[8];
        load8f(x, DSP + ((rb * (D / 32) + c) * 64 + lane) * 8);
        Frag<T> hi, lo;
        split8(x, hi, lo);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          mma(xk[kb][rb], uf, kf[kb][c]);
          mma_hl(dkp[kb][rb], hi, lo, vf[kb][c]);
        }
      }
    }
    Frag<T> kpf[NKB][NRC], dxf[NKB][NRC];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int tok = kvalid[kb] ? krow[kb] : 0;
      const int hw = a.gh * a.gw, pt = tok / hw, rem = tok - pt * hw, py = rem / a.gw, px = rem - py * a.gw;
      float kp[NRB][4], dx[NRB][4];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const int m = 16 * rb + 4 * g + 2 * pr;
          const float2 cs = rope_at<R>(a.rope, a.gt, a.gh, pt, py, px, m / 2);
          const float e0 = xk[kb][rb][2 * pr], e1 = xk[kb][rb][2 * pr + 1];
          const float f0 = elu1(e0), f1 = elu1(e1);
          kp[rb][2 * pr] = f0 * cs.x - f1 * cs.y;
          kp[rb][2 * pr + 1] = f0 * cs.y + f1 * cs.x;
          const float x0 = dkp[kb][rb][2 * pr], x1 = dkp[kb][rb][2 * pr + 1];
          const float d0 = DZ[m] + (x0 * cs.x + x1 * cs.y);
          const float d1 = DZ[m + 1] + (-x0 * cs.y + x1 * cs.x);
          dx[rb][2 * pr] = d0 * (e0 > 0.f ? 1.f : f0);
          dx[rb][2 * pr + 1] = d1 * (e1 > 0.f ? 1.f : f1);
        }
#pragma unroll
      for (int rc = 0; rc < NRC; ++rc) {
        const bool two = 2 * rc + 1 < NRB;
        const int b1 = two ? 2 * rc + 1 : 2 * rc;
        const float keep = two ? 1.f : 0.f;
        pack_rows(kpf[kb][rc], f32x4{kp[2 * rc][0], kp[2 * rc][1], kp[2 * rc][2], kp[2 * rc][3]},
                  f32x4{keep * kp[b1][0], keep * kp[b1][1], keep * kp[b1][2], keep * kp[b1][3]}, 1.f);
        pack_rows(dxf[kb][rc], f32x4{dx[2 * rc][0], dx[2 * rc][1], dx[2 * rc][2], dx[2 * rc][3]},
                  f32x4{keep * dx[b1][0], keep * dx[b1][1], keep * dx[b1][2], keep * dx[b1][3]}, 1.f);
      }
    }
#pragma unroll
    for (int jd = 0; jd < NDB; ++jd) {
      f32x4 av[NKB], ak[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        av[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        ak[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int rc = 0; rc < NRC; ++rc) {
        float x[8];
        load8f(x, DSF + ((size_t)(jd * NRC + rc) * 64 + lane) * 8);
        Frag<T> hi, lo;
        split8(x, hi, lo);
        Frag<T> uf;
        load8(uf, UKP + ((size_t)(jd * NRC + rc) * 64 + lane) * 8);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          mma_hl(av[kb], hi, lo, kpf[kb][rc]);
          mma(ak[kb], uf, dxf[kb][rc]);
        }
      }
      const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float* dko = a.dk + base + (size_t)krow[kb] * D + 16 * jd + 4 * g;
        float* dvo = a.dv + base + (size_t)krow[kb] * D + 16 * jd + 4 * g;
        *reinterpret_cast<float4*>(dko) = kvalid[kb] ? make_float4(ak[kb][0], ak[kb][1], ak[kb][2], ak[kb][3]) : zero;
        *reinterpret_cast<float4*>(dvo) = kvalid[kb] ? make_float4(av[kb][0], av[kb][1], av[kb][2], av[kb][3]) : zero;
      }
    }
  }
}

// bf16 sparse dV and dK in one launch: one block per key tile = 4 waves, each
// holding K and V of its 16 keys and the accumulators of both gradients, over
// the query tiles that keep the key tile (CSC).  Per query tile a wave forms
// S = q k^T and dP = dO v^T, P = exp(scale S - lse) and dS = P (dP - D) scale,
// and adds P^T dO to dV and dS^T q to dK, so the scores and their
// exponentials are computed once per kept pair.  The query-side tiles Q and
// dO are staged once per step for all four waves: both in the layout that
// serves row reads and transposing reads (Q and dO by rows for S and dP,
// both transposed for the two gradient products), both double-buffered, so
// the next query tile's Q, dO, lse and D load during the whole step and one
// barrier per step suffices.
template <int D>
__global__ __launch_bounds__(256, 2) void k_bwd_dkv_bf16(BwdArgs a) {
  constexpr int RB = 2 * D, RG = RB / 16;
  constexpr int NDB = D / 16;
  constexpr int NW = 4;
  constexpr int NI = 64 * RB / 1024 / NW;
  __shared__ __align__(16) uint8_t Qb[2][64 * RB];
  __shared__ __align__(16) uint8_t Gb[2][64 * RB];
  __shared__ __align__(16) float Ls[2][2][64];  // [buffer][lse, D][query]

  const int L = uniform(a.col_order[blockIdx.x]);
  const int bh = uniform(L / a.T), kt = uniform(L - bh * a.T);
  const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const size_t base = (size_t)bh * a.N_pad * D;
  const bf16_t* K = reinterpret_cast<const bf16_t*>(a.k) + base;
  const bf16_t* V = reinterpret_cast<const bf16_t*>(a.v) + base;
  const int nbytes = a.N * RB;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)K, 0, nbytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)V, 0, nbytes, kBufferFlags);
  const i32x4_t qrs = make_rsrc_regs(reinterpret_cast<const bf16_t*>(a.q) + base, nbytes);
  const i32x4_t grs = make_rsrc_regs(reinterpret_cast<const bf16_t*>(a.dout) + base, nbytes);
  // wave 0 stages lse, wave 1 stages D (rows >= N read as 0)
  const i32x4_t srs = make_rsrc_regs(w == 0 ? (const float*)a.lse + (size_t)bh * a.N_pad
                                            : (const float*)a.dsum + (size_t)bh * a.N_pad, a.N * 4);

  const int krow = kt * 64 + 16 * w + l16;
  const bool kvalid = krow < a.N;
  Frag<bf16_t> kf[D / 32], vf[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {  // rows >= N read as zeros
    kf[c].w = __builtin_amdgcn_raw_buffer_load_b128(krs, (krow * D + 32 * c + 8 * g) * 2, 0, 0);
    vf[c].w = __builtin_amdgcn_raw_buffer_load_b128(vrs, (krow * D + 32 * c + 8 * g) * 2, 0, 0);
  }
  f32x4 accv[NDB], acck[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j) {
    accv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    acck[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  if (a.N < 0) { Qb[0][tid] = 0; Qb[1][tid] = 0; Gb[0][tid] = 0; Gb[1][tid] = 0; Ls[0][0][tid & 63] = 0.f; }
  const int beg = a.col_ptr[(size_t)bh * a.T + kt];
  const int end = (int)min((long)a.col_ptr[(size_t)bh * a.T + kt + 1], a.csc_cap);
  const float c2 = a.scale * kLog2e;
  int off[NI];  // Q and dO share the layout, hence the offsets
  dma_offsets_kt<RB, NW>(w, lane, off);
  const int raddr = l16 * RB + 16 * (g ^ swz_kt<RG>(l16));  // row reads
  const int rowl = 4 * g + (l16 >> 2);
  const int taddr = rowl * RB + 16 * (((l16 >> 1) & 1) ^ swz_kt<RG>(rowl)) + 8 * (l16 & 1);  // transposing reads
  int rowv = beg + lane < end ? a.row_idx[beg + lane] : 0;
  int row = __builtin_amdgcn_readlane(rowv, 0);
  int nrow = __builtin_amdgcn_readlane(rowv, 1);
  auto issue = [&](int r, int buf) {
    dma_tile<RB, NW>(qrs, r, off, Qb[buf], w);
    dma_tile<RB, NW>(grs, r, off, Gb[buf], w);
    if (w < 2) lds_dma4(srs, Ls[buf][w], r * 256 + 4 * lane);
  };
  // acc[jd] += (transposed tile tt)^T-part x B fragments over the 32 queries of chunk c
  auto tprod = [&](const uint8_t* tt, const Frag<bf16_t> (&bfr)[2], f32x4 (&acc)[NDB]) {
#pragma unroll
    for (int jd = 0; jd < NDB; ++jd) {
      const int ta = taddr ^ (32 * jd);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        Frag<bf16_t> tf;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const s16x4_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(&tt[ta + (32 * c + 16 * hh) * RB]));
          const uint2 u = __builtin_bit_cast(uint2, t);
          tf.w[2 * hh] = u.x;
          tf.w[2 * hh + 1] = u.y;
        }
        mma(acc[jd], tf, bfr[c]);
      }
    }
  };
  if (beg < end) {
    issue(row, 0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
  }
  for (int j = beg; j < end; ++j) {
    const int cur = (j - beg) & 1;
    const bool more = j + 1 < end;
    if (more) issue(nrow, cur ^ 1);  // that buffer was last read in the previous step
    const uint8_t* Qc = Qb[cur];
    const uint8_t* Gc = Gb[cur];
    Frag<bf16_t> pfr[2], dsfr[2];
    const bool full = row * 64 + 64 <= a.N;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      f32x4 p[2], ds[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int qb = 2 * c + h2;
        f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f}, dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < D / 32; ++cc) {
          Frag<bf16_t> qfr, gfr;
          qfr.w = *reinterpret_cast<const u32x4*>(&Qc[(raddr ^ (64 * cc)) + 16 * RB * qb]);
          gfr.w = *reinterpret_cast<const u32x4*>(&Gc[(raddr ^ (64 * cc)) + 16 * RB * qb]);
          mma(s, qfr, kf[cc]);
          mma(dp, gfr, vf[cc]);
        }
        const float4 l4 = *reinterpret_cast<const float4*>(&Ls[cur][0][16 * qb + 4 * g]);
        const float4 d4 = *reinterpret_cast<const float4*>(&Ls[cur][1][16 * qb + 4 * g]);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
        // query rows >= N read as zeros (Q, dO, lse, D): P = 1 meets a zero dO row in dV,
        // and dS is zeroed there explicitly (only the ragged last tile takes the guard)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -lv[i] * kLog2e));
          p[h2][i] = e;
          ds[h2][i] = e * (dp[i] - dv4[i]) * a.scale;
        }
        if (!full) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (row * 64 + 16 * qb + 4 * g + i >= a.N) ds[h2][i] = 0.f;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      pack_rows(pfr[c], p[0], p[1], 1.f);
      pack_rows(dsfr[c], ds[0], ds[1], 1.f);
    }
    tprod(Gc, pfr, accv);   // dV += P^T dO
    tprod(Qc, dsfr, acck);  // dK += dS^T q
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // this wave's shares of the next Q, dO, lse and D have landed
    lds_barrier();                              // they are visible; every wave is done with this step's tiles
    if (((j + 2 - beg) & 63) == 0 && j + 2 < end) {
      rowv = j + 2 + lane < end ? a.row_idx[j + 2 + lane] : 0;
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    row = nrow;
    nrow = __builtin_amdgcn_readlane(rowv, (j + 2 - beg) & 63);
  }
  if (kvalid) {
    float* ov = a.dv + base + (size_t)krow * D;
    float* ok = a.dk + base + (size_t)krow * D;
#pragma unroll
    for (int jd = 0; jd < NDB; ++jd) {
      float4 x = *reinterpret_cast<float4*>(ov + 16 * jd + 4 * g);
      x.x += accv[jd][0]; x.y += accv[jd][1]; x.z += accv[jd][2]; x.w += accv[jd][3];
      *reinterpret_cast<float4*>(ov + 16 * jd + 4 * g) = x;
      float4 y = *reinterpret_cast<float4*>(ok + 16 * jd + 4 * g);
      y.x += acck[jd][0]; y.y += acck[jd][1]; y.z += acck[jd][2]; y.w += acck[jd][3];
      *reinterpret_cast<float4*>(ok + 16 * jd + 4 * g) = y;
    }
  }
}

// ------------------------------------------------------------- launcher
template <typename T, int D, int R>
static hipError_t bwd_launch_linear(const Shape& s, const BwdArgs& a, hipStream_t st) {
  hipError_t e;
  k_bwd_q<T, D, R><<<8 * ((a.nchunk + 1) / 2) * ((s.B * s.H + 7) / 8), 512, 0, st>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  k_bwd_fin<T, D, R><<<dim3(s.B * s.H, R / 8), 256, 0, st>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  k_bwd_k<T, D, R><<<dim3((a.T + a.tpc_k - 1) / a.tpc_k, s.B * s.H), 512, 0, st>>>(a);
  return hipGetLastError();
}

template <typename T>
static hipError_t bwd_linear_by_shape(const Shape& s, const BwdArgs& a, hipStream_t st) {
  if (s.d == 64) {
    if (s.rank == 16) return bwd_launch_linear<T, 64, 16>(s, a, st);
    if (s.rank == 32) return bwd_launch_linear<T, 64, 32>(s, a, st);
    return bwd_launch_linear<T, 64, 64>(s, a, st);
  }
  if (s.rank == 16) return bwd_launch_linear<T, 128, 16>(s, a, st);
  if (s.rank == 32) return bwd_launch_linear<T, 128, 32>(s, a, st);
  return bwd_launch_linear<T, 128, 64>(s, a, st);
}

// CSC of the mask, then the sparse dQ and dK/dV kernels.  csc_cnt: [BH*T]
// scratch; col_ptr [BH*T + 1]; row_idx capacity `cap`.
template <typename T>
static hipError_t bwd_sparse(const Shape& s, BwdArgs a, int32_t* csc_cnt, int32_t* col_ptr, int32_t* row_idx,
                             uint32_t* bits, long cap, hipStream_t st) {
  hipError_t e;
  const int rows = s.B * s.H * s.T, W = (s.T + 31) / 32;
  const long nbits = (long)rows * W;
  k_zero_i32<<<(int)((nbits + 255) / 256), 256, 0, st>>>((int)nbits, reinterpret_cast<int32_t*>(bits));
  k_csc_bits<<<(rows + 255) / 256, 256, 0, st>>>(rows, s.T, W, a.row_ptr, a.col_idx, bits);
  k_csc_cols<false><<<(rows + 255) / 256, 256, 0, st>>>(rows, W, bits, csc_cnt, nullptr, nullptr, cap);
  k_csc_scan<<<1, 1024, 0, st>>>(rows, csc_cnt, col_ptr);
  k_csc_cols<true><<<(rows + 255) / 256, 256, 0, st>>>(rows, W, bits, nullptr, col_ptr, row_idx, cap);
  // the counts are no longer needed: their buffer takes the dK / dV order
  if (s.T <= kOrderMaxT)
    k_csc_order<<<s.B * s.H, 1024, 0, st>>>(s.T, col_ptr, cap, csc_cnt);
  else
    k_iota_i32<<<(rows + 255) / 256, 256, 0, st>>>(rows, csc_cnt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  a.col_ptr = col_ptr;
  a.row_idx = row_idx;
  a.csc_cap = cap;
  a.col_order = csc_cnt;
  const long grid = 8 * (a.nrows / a.T) * ((a.T + 7) / 8);
  if constexpr (sizeof(T) == 2) {
    if (s.d == 64) k_bwd_dq_bf16<64, 4><<<grid, 256, 0, st>>>(a);
    else k_bwd_dq_bf16<128, 4><<<grid, 256, 0, st>>>(a);
  } else {
    if (s.d == 64) k_bwd_dq<T, 64><<<grid, 256, 0, st>>>(a);
    else k_bwd_dq<T, 128><<<grid, 256, 0, st>>>(a);
  }
  if constexpr (sizeof(T) == 2) {
    if (s.d == 64) k_bwd_dkv_bf16<64><<<rows, 256, 0, st>>>(a);
    else k_bwd_dkv_bf16<128><<<rows, 256, 0, st>>>(a);
  } else {
    if (s.d == 64) k_bwd_dkv<T, 64><<<grid, 256, 0, st>>>(a);
    else k_bwd_dkv<T, 128><<<grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_f32(const Shape& s, const BwdArgs& a, int32_t* csc_cnt, int32_t* col_ptr, int32_t* row_idx,
                          uint32_t* bits, long cap, bool linear_part, hipStream_t st);

}  // namespace hsa
