// Kernels of the streaming pass over K and V (one read of each) and the finalize step of the
// linear branch.
//
//  * Tile pooling of K: float64 column sums of the valid rows of every 64-token
//    tile, divided by the valid count (the mean-pooled tile statistic used to
//    find the high-energy tiles; SparkDiffusion news article, section 05), also
//    split into bf16 hi + lo parts for the selection's matrix-core scores.  The
//    query tiles are pooled by the selection kernel itself.
//  * Linear key/value state of the rotary low-rank branch (same section: a
//    low-rank linear branch with rotary position information):
//      F = K U_k (matrix cores), phi = elu(F) + 1, z += sum_j phi_j,
//      k'_j = rope(phi_j, p_j),  S^T += V^T k'  (matrix cores, contraction
//      over tokens).  Each block writes one partial (S, z); the finalize kernel
//      adds the partials in a fixed order, so results are bitwise reproducible.
//
// The pass is HBM-bound: every element of K and V is read once with 16-byte
// loads, the next tile is prefetched into registers while the current one is
// processed, and all arithmetic runs from LDS and registers.
#pragma once
#include <type_traits>
#include "common.hpp"
#include "kernels.hpp"

namespace hsa {

// ----------------------------------------------------------------- RoPE table
static __global__ void k_rope_table(int gt, int gh, int gw, int rank, double base, float2* tab) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  int dims[3] = {3 * rank / 8, 3 * rank / 8, rank / 4};
  int sizes[3] = {gt, gh, gw};
  int off = 0;
  for (int ax = 0; ax < 3; ++ax) {
    int half = dims[ax] / 2, n = sizes[ax] * half;
    if (i < off + n) {
      int j = i - off, pos = j / half, m = j % half;
      double theta = pow(base, -2.0 * (double)m / (double)dims[ax]);
      double ang = (double)pos * theta;
      tab[i] = make_float2((float)cos(ang), (float)sin(ang));
      return;
    }
    off += n;
  }
}

// Location of feature pair jp (0 .. r/2-1) in the RoPE table: axis, m and the
// table offset of that axis.
struct RopeSlot { int axis, m, half, off; };
__device__ __forceinline__ RopeSlot rope_slot(int jp, int rank, int gt, int gh) {
  int ht = 3 * rank / 16, hh = 3 * rank / 16, hw = rank / 8;  // pairs per axis
  RopeSlot s;
  if (jp < ht) { s.axis = 0; s.m = jp; s.half = ht; s.off = 0; }
  else if (jp < ht + hh) { s.axis = 1; s.m = jp - ht; s.half = hh; s.off = gt * ht; }
  else { s.axis = 2; s.m = jp - ht - hh; s.half = hw; s.off = gt * ht + gh * hh; }
  return s;
}

typedef short s16x4_lds_t __attribute__((ext_vector_type(4)));

// Value of the neighbouring lane in the pair (2m, 2m + 1): a DPP quad
// permutation (1, 0, 3, 2), no LDS traffic.
__device__ __forceinline__ float quad_swap1(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}

// ------------------------------------------------------ operand conversions
template <typename T, typename OT> struct Conv;
// Same type: raw copy.
template <typename T> struct Conv<T, T> {
  __device__ static void row(T* dst, const Chunk8<T>& c);
};
template <> __device__ void Conv<bf16_t, bf16_t>::row(bf16_t* dst, const Chunk8<bf16_t>& c) {
  *reinterpret_cast<u32x4*>(dst) = c.w;
}
template <> __device__ void Conv<float, float>::row(float* dst, const Chunk8<float>& c) {
  reinterpret_cast<float4*>(dst)[0] = c.a;
  reinterpret_cast<float4*>(dst)[1] = c.b;
}
// FP8 codes -> exact bf16 values (E4M3 values fit bf16's 8-bit significand).
template <> struct Conv<fp8_t, bf16_t> {
  __device__ static void row(bf16_t* dst, const Chunk8<fp8_t>& c) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(elem(c, 2 * j), elem(c, 2 * j + 1));
    *reinterpret_cast<u32x4*>(dst) = w;
  }
};

// Write 4 consecutive values of operand type at dst.
__device__ __forceinline__ void st4(bf16_t* dst, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}
__device__ __forceinline__ void st4(float* dst, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
}

// Position of key k (0..63) of a tile inside the transposed V layout used
// as the A operand of a contraction over tokens: within each 32-key chunk,
// key 16h + 4g + i sits at 8g + 4h + i, so that lane group g reads its eight
// contraction slots with one 16-byte load.
__device__ __forceinline__ int vt_pos(int key) {
  int c = key >> 5, kk = key & 31;
  int h = kk >> 4, g = (kk >> 2) & 3, i = kk & 3;
  return 32 * c + 8 * g + 4 * h + i;
}

// fp8 V^T tiles for the sparse kernel: vt8[d][p] = code of V[key][d] with
// key = 16 kb + 4 g + i stored at p = 16 g + 4 kb + i, so that lane group g of
// a 16x16x128 operand reads its 16 keys of a tile as one 16-byte run.
inline __device__ __forceinline__ int vt8_pos(int key) {
  const int kb = key >> 4, g = (key >> 2) & 3, i = key & 3;
  return 16 * g + 4 * kb + i;
}

// Thread `u` (< 16 * D / 8) holds codes of keys 4(u%16) .. +3 for dims
// 8(u/16) .. +7 and writes them, transposed, into an LDS tile of D rows x 80 B.
inline __device__ __forceinline__ void stage_vt8(uint8_t* Vt8, int u, const Chunk8<fp8_t>* vc) {
  const int kg = u % 16, c8 = u / 16;
  const int p0 = vt8_pos(4 * kg);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int sh = 8 * (e & 3);
    uint32_t w = 0;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const uint32_t word = (e < 4) ? vc[ii].w.x : vc[ii].w.y;
      w |= ((word >> sh) & 0xFFu) << (8 * ii);
    }
    *reinterpret_cast<uint32_t*>(&Vt8[(c8 * 8 + e) * 80 + p0]) = w;
  }
}

// Copy a staged fp8 V^T tile (D rows x 64 codes) to global memory.
template <int D = 128>
__device__ __forceinline__ void write_vt8(uint8_t* dst, const uint8_t* Vt8, int tid) {
  for (int q = tid; q < D * 4; q += 256) {
    const int row = q >> 2, part = q & 3;
    *reinterpret_cast<u32x4*>(dst + row * 64 + part * 16) = *reinterpret_cast<const u32x4*>(&Vt8[row * 80 + part * 16]);
  }
}

// --------------------------------------------------------- streaming pass
struct StreamArgs {
  int N, N_pad, T, nchunk, tpc;
  int gt, gh, gw;
  const void* q;
  const void* k;
  const void* v;
  const float* qs;
  const float* ks;
  const float* vs;
  const void* uk;  // [H][d][r] in the parameter type
  int H;
  double* kmean;  // [BH][T][d] tile means of K
  uint16_t* khi;  // bf16 hi part of the means, in fragment order (kfrag_index)
  uint16_t* klo;  // bf16 lo part (mean - hi, rounded), the same order
  double* kbar_out;
  float* part_s;
  float* part_z;
  const float2* rope;
  int nrope;  // RoPE table entries
  void* vt;  // optional: V tiles transposed, [BH][T][d][64] with keys permuted as in LDS
  void* tile_s;   // with TILES: [BH][T] state of each tile alone as readout A fragments (parameter type)
  float* tile_z;  // with TILES: [BH][T][r] feature sum of each tile alone
};

// RoPE tables up to this many entries (11.5 KB at 720P, rank 64) are staged
// in LDS once per block, so the per-token lookups are LDS reads (two blocks
// per CU still fit: at most ~75 KB each, for fp8 inputs with d = 128).
constexpr int kRopeLdsMax = 1536;

// TILES: also write every tile's own state and feature sum (the partial
// state of the block is then their sum).  The state product then runs with
// swapped operands, S = k'^T V, so that each lane holds 4 consecutive ranks
// of one d column: exactly 4 consecutive slots of a readout A fragment of
// S^T (d rows, contraction over r), written with one store.
template <typename T, typename OT, int D, int R, bool POOL, bool STATE, bool RLDS = false, bool TILES = false>
__global__ __launch_bounds__(256, 2) void k_stream(StreamArgs a) {
  constexpr int CPR = D / 8;              // 8-element chunks per row
  constexpr int NCONT = 256 / CPR;        // threads sharing a column chunk
  constexpr int KCH = 64 * CPR / 256;     // row chunks per thread per tile
  constexpr int NVU = 16 * CPR;           // V units (4 keys x 8 dims)
  constexpr int KSTR = D + 8;             // LDS row stride of K (elements)
  constexpr int VSTR = 64 + 8;            // LDS row stride of V^T
  // bf16 inputs keep V row-major in LDS and read V^T operands with
  // transposing reads; the other types stage V transposed
  constexpr bool VROW = std::is_same<T, bf16_t>::value;
  constexpr int VRS = D + 16;             // LDS row stride of row-major V (rows 8 banks apart)
  constexpr int NRB = R / 16;             // 16-wide blocks of the rank
  constexpr int NDG = 4 / NRB;            // waves sharing an r block
  constexpr int DBW = (D / 16) / NDG;     // 16-wide d blocks per wave
  static_assert(R == 16 || R == 32 || R == 64, "rank");
  static_assert(D == 64 || D == 128, "head dim");

  __shared__ __align__(16) OT Ks[STATE ? 64 * KSTR : 1];
  __shared__ __align__(16) OT Vt[(STATE && !VROW) ? D * VSTR : 1];
  __shared__ __align__(16) OT Vr[(STATE && VROW) ? 64 * VRS : 1];
  __shared__ __align__(16) uint8_t Vt8[(STATE && sizeof(T) == 1) ? D * 80 : 16];  // fp8 V^T tile for the sparse kernel
  __shared__ double redk[POOL ? NCONT * D : 1];
  // per token of the current tile: the RoPE table row of its position on each
  // axis (the axis's offset in the table + position x pairs of the axis)
  __shared__ __align__(16) int sofs[3][64];
  __shared__ float2 rtab[RLDS ? kRopeLdsMax : 1];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int h = bh % a.H;
  const int t0 = chunk * a.tpc;
  const int t1 = min(a.T, t0 + a.tpc);
  if (t0 >= t1) return;

  const size_t base = (size_t)bh * a.N_pad * D;
  const T* K = reinterpret_cast<const T*>(a.k) + base;
  const T* V = reinterpret_cast<const T*>(a.v) + base;
  const int col8 = tid % CPR;
  const int row0 = tid / CPR;

  // per-wave linear-branch constants
  const int rb = w % NRB, dg = w / NRB;
  const int r = 16 * rb + l16;
  Frag<OT> uf[D / 32];
  RopeSlot rs;
  const int* sax = nullptr;  // this lane's axis row of sofs, from token 4 g
  float zacc = 0.f;
  f32x4 accS[DBW];
  if constexpr (STATE) {
    const OT* U = reinterpret_cast<const OT*>(a.uk) + (size_t)h * D * R;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      float tmp[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const OT* p = U + (size_t)(32 * c + 8 * g + s) * R + r;
        if constexpr (sizeof(OT) == 4) tmp[s] = *reinterpret_cast<const float*>(p);
        else tmp[s] = bf16_bits_to_f32(reinterpret_cast<const bf16_t*>(p)->bits);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) uf[c].set_pair(j, tmp[2 * j], tmp[2 * j + 1]);
    }
    rs = rope_slot(r >> 1, R, a.gt, a.gh);
    if constexpr (RLDS) {
      for (int i = tid; i < a.nrope; i += 256) rtab[i] = a.rope[i];  // published by the loop's first barrier
    }
    sax = &sofs[rs.axis][4 * g];
#pragma unroll
    for (int j = 0; j < DBW; ++j) accS[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // buffer views of this head's valid rows: rows >= N read as zeros
  const int nbytes = a.N * D * (int)sizeof(T);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(K, nbytes), vrs = make_rsrc(V, nbytes);
  // Two tiles in flight per block: while tile t is processed from one
  // register set, tile t + 1 is already loading into the other, and tile t + 2
  // is issued into the first set once tile t sits in LDS.  Every step issues
  // the same loads (a tile past the chunk has an index beyond T, which reads
  // zeros from the bounds-checked views and moves no data), so that the
  // compiler can count the loads in flight and waits for the current tile
  // only.  fp8 inputs load their per-tile scales with the tile.
  constexpr bool SCALED = sizeof(T) == 1;
  struct TileRegs { Chunk8<T> k[KCH], v[VROW ? KCH : 4]; float sk, sv; };
  TileRegs tra, trb;
  const size_t sbase = (size_t)bh * a.T;
  auto load_tile = [&](int t, TileRegs& c) {
    if constexpr (SCALED) {  // (scales exist for every fp8 tensor a step reads)
      const size_t i = sbase + min(t, a.T - 1);
      c.sk = a.ks[i];
      if constexpr (STATE) c.sv = a.vs[i];
    }
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int e = (t * 64 + row0 + i * NCONT) * D + col8 * 8;
      bload8(c.k[i], krs, e);
    }
    if constexpr (STATE && VROW) {
#pragma unroll
      for (int i = 0; i < KCH; ++i) bload8(c.v[i], vrs, (t * 64 + row0 + i * NCONT) * D + col8 * 8);
    } else if constexpr (STATE) {
      if (tid < NVU) {
        const int kg = tid % 16, c8 = tid / 16;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) bload8(c.v[ii], vrs, (t * 64 + 4 * kg + ii) * D + c8 * 8);
      }
    }
  };

  auto process = [&](int t, TileRegs& c) {
    const bool live = t < t1;  // false: a step past the chunk, which only issues its loads
    // this tile's scales, taken before the registers are reloaded
    const float tsk = SCALED ? c.sk : 1.f, tsv = SCALED && STATE ? c.sv : 1.f;
    if (live) {
      // ---- registers -> LDS
      if constexpr (POOL) {
        double pk[8];
  #pragma unroll
        for (int e = 0; e < 8; ++e) pk[e] = 0.0;
  #pragma unroll
        for (int i = 0; i < KCH; ++i)
  #pragma unroll
          for (int e = 0; e < 8; ++e) pk[e] += (double)elem(c.k[i], e);
  #pragma unroll
        for (int e = 0; e < 8; ++e) redk[row0 * D + col8 * 8 + e] = pk[e];
      }
      if constexpr (STATE) {
  #pragma unroll
        for (int i = 0; i < KCH; ++i) Conv<T, OT>::row(&Ks[(row0 + i * NCONT) * KSTR + col8 * 8], c.k[i]);
        if constexpr (VROW) {
  #pragma unroll
          for (int i = 0; i < KCH; ++i) Conv<T, OT>::row(&Vr[(row0 + i * NCONT) * VRS + col8 * 8], c.v[i]);
        } else if (tid < NVU) {
          int kg = tid % 16, c8 = tid / 16;
          int p0 = vt_pos(4 * kg);
  #pragma unroll
          for (int e = 0; e < 8; ++e)
            st4(&Vt[(c8 * 8 + e) * VSTR + p0], elem(c.v[0], e), elem(c.v[1], e), elem(c.v[2], e), elem(c.v[3], e));
        }
        if (tid < 64) {
          const int tok = min(t * 64 + tid, a.N - 1), hw = a.gh * a.gw;
          const int pt = tok / hw, rem = tok - pt * hw;
          const int ph = rem / a.gw, pw = rem - ph * a.gw;
          constexpr int PT = 3 * R / 16, PH = 3 * R / 16, PW = R / 8;  // RoPE pairs per axis
          sofs[0][tid] = pt * PT;
          sofs[1][tid] = a.gt * PT + ph * PH;
          sofs[2][tid] = a.gt * PT + a.gh * PH + pw * PW;
        }
        if constexpr (sizeof(T) == 1) {
          if (a.vt && tid < NVU) stage_vt8(Vt8, tid, c.v);
        }
      }
      __syncthreads();
    }
    load_tile(t + 2 < t1 ? t + 2 : a.T + 1, c);
    if (live) {
      if constexpr (STATE && sizeof(T) == 1) {
        // hand the transposed fp8 tile to the sparse kernel
        if (a.vt) write_vt8(reinterpret_cast<uint8_t*>(a.vt) + ((size_t)bh * a.T + t) * D * 64, Vt8, tid);
      }

      if constexpr (STATE) {
        const float sk = tsk, sv = tsv;
        f32x4 accF[4];
  #pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          accF[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
          for (int c = 0; c < D / 32; ++c) {
            Frag<OT> kf;
            load8(kf, &Ks[(16 * tb + l16) * KSTR + 32 * c + 8 * g]);
            mma(accF[tb], kf, uf[c]);
          }
        }
        float kp[4][4];
        float ztile = 0.f;  // this lane's share of the tile's feature sum
        float phi[4][4];
  #pragma unroll
        for (int tb = 0; tb < 4; ++tb)
  #pragma unroll
          for (int i = 0; i < 4; ++i) phi[tb][i] = elu1(accF[tb][i] * sk);
        if (__builtin_expect(t * 64 + 64 > a.N, 0)) {  // ragged last tile: tokens past N add nothing
  #pragma unroll
          for (int tb = 0; tb < 4; ++tb)
  #pragma unroll
            for (int i = 0; i < 4; ++i)
              if (t * 64 + 16 * tb + 4 * g + i >= a.N) phi[tb][i] = 0.f;
        }
  #pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          // table rows of this lane's four tokens 16 tb + 4 g + i on its axis
          const int4 ro = *reinterpret_cast<const int4*>(sax + 16 * tb);
          const int rows[4] = {ro.x, ro.y, ro.z, ro.w};
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float f = phi[tb][i];
            if constexpr (TILES) ztile += f;
            else zacc += f;
            const float other = quad_swap1(f);  // the feature paired with this lane's by RoPE
            const float2 cs = RLDS ? rtab[rows[i] + rs.m] : a.rope[rows[i] + rs.m];
            float rot = (r & 1) ? (other * cs.y + f * cs.x) : (f * cs.x - other * cs.y);
            kp[tb][i] = rot * sv;
          }
        }
        if constexpr (TILES) {
          zacc += ztile;
          const float zt = group4_sum(ztile);
          if (dg == 0 && g == 0) a.tile_z[((size_t)bh * a.T + t) * R + r] = zt;
        }
        Frag<OT> kf2[2];
  #pragma unroll
        for (int c = 0; c < 2; ++c) {
          kf2[c].set_pair(0, kp[2 * c][0], kp[2 * c][1]);
          kf2[c].set_pair(1, kp[2 * c][2], kp[2 * c][3]);
          kf2[c].set_pair(2, kp[2 * c + 1][0], kp[2 * c + 1][1]);
          kf2[c].set_pair(3, kp[2 * c + 1][2], kp[2 * c + 1][3]);
        }
        f32x4 accT[TILES ? DBW : 1];
        if constexpr (TILES) {
  #pragma unroll
          for (int j = 0; j < DBW; ++j) accT[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
  #pragma unroll
        for (int j = 0; j < DBW; ++j) {
          int db = dg * DBW + j;
  #pragma unroll
          for (int c = 0; c < 2; ++c) {
            Frag<OT> vf;
            if constexpr (VROW) {
              // slot s of lane group g holds token 32c + 16(s/4) + 4g + s%4 (as kf2)
  #pragma unroll
              for (int hh = 0; hh < 2; ++hh) {
                const int row = 32 * c + 16 * hh + 4 * g + (l16 >> 2), col = 16 * db + 4 * (l16 & 3);
                typedef __attribute__((address_space(3))) s16x4_lds_t s16x4_as3;
                const s16x4_lds_t t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_as3*)(&Vr[row * VRS + col]));
                const uint2 u = __builtin_bit_cast(uint2, t4);
                vf.w[2 * hh] = u.x;
                vf.w[2 * hh + 1] = u.y;
              }
            } else {
              load8(vf, &Vt[(16 * db + l16) * VSTR + 32 * c + 8 * g]);
            }
            if constexpr (TILES) mma(accT[j], kf2[c], vf);
            else mma(accS[j], vf, kf2[c]);
          }
        }
        if constexpr (TILES) {
          // the tile's own S block: column d = 16 db + l16, ranks 16 rb + 4 g .. + 3,
          // i.e. fragment (db, rb / 2), lane l16 + 16 g, slots 4 (rb % 2) .. + 3
          constexpr int NRC = (R + 31) / 32, NFE = (D / 16) * NRC * 512;
          OT* ts = reinterpret_cast<OT*>(a.tile_s) + ((size_t)bh * a.T + t) * NFE;
  #pragma unroll
          for (int j = 0; j < DBW; ++j) {
            const int db = dg * DBW + j;
            OT* dst = ts + ((db * NRC + (rb >> 1)) * 64 + l16 + 16 * g) * 8 + 4 * (rb & 1);
            st4(dst, accT[j][0], accT[j][1], accT[j][2], accT[j][3]);
            if constexpr (R % 32 != 0) st4(dst + 4, 0.f, 0.f, 0.f, 0.f);  // rank 16: no upper half
            accS[j] += accT[j];
          }
        }
      }
      if constexpr (POOL) {
        // thread tid < D: column tid of K
        if (tid < D) {
          double sum = 0.0;
  #pragma unroll
          for (int c = 0; c < NCONT; ++c) sum += redk[c * D + tid];
          if constexpr (SCALED) sum *= (double)tsk;
          // a full tile divides by 64, exactly a multiply by 2^-6
          const int cnt = min(64, a.N - t * 64);
          const double mean = cnt == 64 ? sum * 0.015625 : sum / (double)cnt;
          const size_t o = ((size_t)bh * a.T + t) * D + tid;  // one 1 KB row per tile
          a.kmean[o] = mean;
          if (a.kbar_out) a.kbar_out[o] = mean;
          const uint32_t hb = f32_to_bf16_bits((float)mean);
          const size_t of = (size_t)bh * kfrag_tiles(a.T) * D + kfrag_index(t, tid, D);  // fragment order
          a.khi[of] = (uint16_t)hb;
          a.klo[of] = (uint16_t)f32_to_bf16_bits((float)(mean - (double)bf16_bits_to_f32(hb)));
        }
      }
      __syncthreads();
    }
  };

  // (in this order: the loop expects the loads of tra to be the older ones,
  // and the compiler's wait counts at the loop head cover both ways in)
  load_tile(t0, tra);
  __builtin_amdgcn_sched_barrier(0);
  load_tile(t0 + 1 < t1 ? t0 + 1 : a.T + 1, trb);
  __builtin_amdgcn_sched_barrier(0);
  for (int t = t0; t < t1; t += 2) {
    process(t, tra);
    process(t + 1, trb);
  }
  if constexpr (POOL) {  // the padding of the last key block of the hi / lo parts reads as zero
    if (t1 == a.T && tid < D) {
      for (int t = a.T; t < kfrag_tiles(a.T); ++t) {
        const size_t of = (size_t)bh * kfrag_tiles(a.T) * D + kfrag_index(t, tid, D);
        a.khi[of] = 0;
        a.klo[of] = 0;
      }
    }
  }

  if constexpr (STATE) {
    const size_t pbase = ((size_t)bh * a.nchunk + chunk);
#pragma unroll
    for (int j = 0; j < DBW; ++j) {
      int db = dg * DBW + j;
      if constexpr (TILES) {  // swapped layout: column d = 16 db + l16, ranks 16 rb + 4 g + i
#pragma unroll
        for (int i = 0; i < 4; ++i) a.part_s[(pbase * R + 16 * rb + 4 * g + i) * D + 16 * db + l16] = accS[j][i];
      } else {
        *reinterpret_cast<float4*>(&a.part_s[(pbase * R + r) * D + 16 * db + 4 * g]) =
            make_float4(accS[j][0], accS[j][1], accS[j][2], accS[j][3]);
      }
    }
    float zt = group4_sum(zacc);
    if (dg == 0 && g == 0) a.part_z[pbase * R + r] = zt;
  }
}

// ------------------------------------------------------------- V transpose
// fp8 V^T tiles for the sparse kernel when no streaming pass runs (sparse
// attention on a given CSR).  One block per (tile, b*H + h); rows past N are
// zero codes.
static __global__ __launch_bounds__(256) void k_vtranspose_fp8(int N, int N_pad, int T, const fp8_t* __restrict__ v,
                                                        uint8_t* __restrict__ vt) {
  constexpr int D = 128;
  __shared__ __align__(16) uint8_t Vt8[D * 80];
  const int t = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const fp8_t* V = v + (size_t)bh * N_pad * D;
  Chunk8<fp8_t> c[4];
  const int kg = tid % 16, c8 = tid / 16;
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int gr = t * 64 + 4 * kg + ii;
    if (gr < N) gload8(c[ii], V + (size_t)gr * D + c8 * 8);
    else zero8(c[ii]);
  }
  stage_vt8(Vt8, tid, c);
  __syncthreads();
  write_vt8(vt + ((size_t)bh * T + t) * D * 64, Vt8, tid);
}

// ------------------------------------------------------------- finalize
// Per (b, h) and slice of 8 rank rows: S = sum of the partial states (fixed
// order), S' = S W_o, written as readout A fragments (float, or bf16 hi + lo);
// the first slice also writes z and zero-fills the fragment slots past r, and
// the first slice of each head of batch 0 writes U_q^T as A fragments.
struct FinalArgs {
  int nchunk, H, B;
  const float* part_s;
  const float* part_z;
  const void* wo;   // [H][d][d]
  const void* uq;   // [H][d][r]
  void* sp_frag;
  float* z;
  void* uq_frag;
  float* s_full;   // optional: [BH] S itself (before W_o) as float readout A fragments
  float* s_pfrag;  // optional (backward): [BH][r*d] S itself (before W_o), perm_frag_index order
  void* wob_frag;  // optional (backward): [H] W_o as A fragments
  void* uqp_frag;  // optional (backward): [H] U_q in perm_frag_index order
  void* wo_frag;   // optional: [H] W_o^T as A fragments
};

constexpr int kFinRows = 8;  // rank rows per finalize block

template <typename OT>
__device__ __forceinline__ float ld_param(const OT* p, size_t i) {
  if constexpr (sizeof(OT) == 4) return reinterpret_cast<const float*>(p)[i];
  else return bf16_bits_to_f32(reinterpret_cast<const bf16_t*>(p)[i].bits);
}

template <typename OT, int D, int R>
__device__ __forceinline__ void put_sp(void* frag, size_t bh, int rr, int e, float x) {
  constexpr int NRC = (R + 31) / 32;
  constexpr int NFE = (D / 16) * NRC * 512;
  const size_t idx = sp_frag_index<D, R>(rr, e);
  if constexpr (sizeof(OT) == 4) {
    reinterpret_cast<float*>(frag)[bh * NFE + idx] = x;
  } else {
    uint16_t hi = (uint16_t)f32_to_bf16_bits(x);
    uint16_t lo = (uint16_t)f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
    uint16_t* out = reinterpret_cast<uint16_t*>(frag) + bh * 2 * NFE;
    out[idx] = hi;
    out[NFE + idx] = lo;
  }
}

template <typename OT, int D, int R>
__global__ __launch_bounds__(256) void k_finalize(FinalArgs a) {
  constexpr int NRB = R / 16;
  constexpr int NRC = (R + 31) / 32;
  __shared__ float S[kFinRows * D];
  const int tid = threadIdx.x, bh = blockIdx.x, h = bh % a.H;
  const int r0 = blockIdx.y * kFinRows;
  const float* ps = a.part_s + (size_t)bh * a.nchunk * R * D + (size_t)r0 * D;
  for (int e = tid; e < kFinRows * D; e += 256) {
    float s = 0.f;
    for (int c = 0; c < a.nchunk; ++c) s += ps[(size_t)c * R * D + e];
    S[e] = s;
  }
  if (blockIdx.y == 0 && tid < R) {
    float s = 0.f;
    for (int c = 0; c < a.nchunk; ++c) s += a.part_z[((size_t)bh * a.nchunk + c) * R + tid];
    a.z[(size_t)bh * R + tid] = s;
  }
  __syncthreads();
  if (a.s_pfrag) {
    for (int e = tid; e < kFinRows * D; e += 256)
      a.s_pfrag[(size_t)bh * R * D + perm_frag_index(r0 + e / D, e % D, D)] = S[e];
    if (blockIdx.y == 0 && bh < a.H) {
      // W_o A fragments: frag (jd, cc), lane l, slot s -> W_o[16 jd + l%16][32 cc + 8 (l/16) + s]
      const OT* W = reinterpret_cast<const OT*>(a.wo) + (size_t)h * D * D;
      OT* wout = reinterpret_cast<OT*>(a.wob_frag) + (size_t)h * D * D;
      for (int idx = tid; idx < D * D; idx += 256) {
        const int s2 = idx & 7, l = (idx >> 3) & 63, fr = idx >> 9;
        const int cc = fr % (D / 32), jd = fr / (D / 32);
        wout[idx] = W[(size_t)(16 * jd + (l & 15)) * D + 32 * cc + 8 * (l >> 4) + s2];
      }
      const OT* U = reinterpret_cast<const OT*>(a.uq) + (size_t)h * D * R;
      OT* uout = reinterpret_cast<OT*>(a.uqp_frag) + (size_t)h * (D / 16) * NRC * 512;
      for (int idx = tid; idx < (D / 16) * NRC * 512; idx += 256) {
        int rr, cc;
        perm_frag_source(idx, R, &rr, &cc);
        uout[idx] = cc < R ? U[(size_t)rr * R + cc] : OT{};
      }
    }
  }
  if (a.s_full) {
    constexpr int NFE = (D / 16) * NRC * 512;
    float* sf = a.s_full + (size_t)bh * NFE;
    for (int e = tid; e < kFinRows * D; e += 256) sf[sp_frag_index<D, R>(r0 + e / D, e % D)] = S[e];
    if (blockIdx.y == 0)  // rank 16: the upper half of each 32-row chunk is zero
      for (int e = tid; e < (32 * NRC - R) * D; e += 256) sf[sp_frag_index<D, R>(R + e / D, e % D)] = 0.f;
  }
  const OT* W = reinterpret_cast<const OT*>(a.wo) + (size_t)h * D * D;
  constexpr int PER = kFinRows * D / 256;  // outputs per thread
  const int col = tid % D;
  const int rbase = tid / D;
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  for (int d = 0; d < D; ++d) {
    const float wv = ld_param(W, (size_t)d * D + col);
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = fmaf(S[(rbase + j * (256 / D)) * D + d], wv, acc[j]);
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) put_sp<OT, D, R>(a.sp_frag, bh, r0 + rbase + j * (256 / D), col, acc[j]);
  if (blockIdx.y == 0) {
    // fragment slots of rank rows R .. 32*NRC-1 (rank 16 only) stay zero
    for (int e = tid; e < (32 * NRC - R) * D; e += 256) put_sp<OT, D, R>(a.sp_frag, bh, R + e / D, e % D, 0.f);
    // U_q^T fragments: frag (rb, c), lane l, slot s -> U_q[d][r] with
    // r = 16 rb + l%16, d = 32 c + 8 (l/16) + s.
    if (bh < a.H) {
      const int nue = NRB * (D / 32) * 64 * 8;
      const OT* U = reinterpret_cast<const OT*>(a.uq) + (size_t)h * D * R;
      OT* out = reinterpret_cast<OT*>(a.uq_frag) + (size_t)h * nue;
      for (int idx = tid; idx < nue; idx += 256) {
        int s2 = idx & 7, l = (idx >> 3) & 63, fr = idx >> 9;
        int c = fr % (D / 32), rbk = fr / (D / 32);
        int rr = 16 * rbk + (l & 15), d = 32 * c + 8 * (l >> 4) + s2;
        out[idx] = U[(size_t)d * R + rr];
      }
      // W_o^T fragments for O_lW^T = W_o^T O_l^T: frag (jo, c), lane l, slot
      // s -> W_o[i][o] with o = 16 jo + l%16 and i = 16 (2c + s/4) + 4 (l/16)
      // + s%4, the order in which accumulator columns pack into B fragments.
      if (a.wo_frag) {
        constexpr int nwe = (D / 16) * (D / 32) * 512;
        OT* wout = reinterpret_cast<OT*>(a.wo_frag) + (size_t)h * nwe;
        for (int idx = tid; idx < nwe; idx += 256) {
          const int s2 = idx & 7, l = (idx >> 3) & 63, fr = idx >> 9;
          const int c = fr % (D / 32), jo = fr / (D / 32);
          const int i = 16 * (2 * c + (s2 >> 2)) + 4 * (l >> 4) + (s2 & 3), o = 16 * jo + (l & 15);
          wout[idx] = W[(size_t)i * D + o];
        }
      }
    }
  }
}

// Launch helpers shared by the bf16/fp8 translation unit and the float32 one.
template <typename T, typename OT, int D, int R>
static hipError_t stream_dispatch(const Shape& s, const StreamArgs& a, bool pool, bool state, hipStream_t st) {
  dim3 grid(a.nchunk, s.B * s.H);
  // (the fp8 variant's LDS is already full with its two V^T tiles)
  const bool rlds = a.nrope <= kRopeLdsMax;
  if (state && a.tile_s) {  // per-tile states for the complement variant
    if (pool && rlds) k_stream<T, OT, D, R, true, true, true, true><<<grid, 256, 0, st>>>(a);
    else if (pool) k_stream<T, OT, D, R, true, true, false, true><<<grid, 256, 0, st>>>(a);
    else if (rlds) k_stream<T, OT, D, R, false, true, true, true><<<grid, 256, 0, st>>>(a);
    else k_stream<T, OT, D, R, false, true, false, true><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
  }
  if (pool && state && rlds) k_stream<T, OT, D, R, true, true, true><<<grid, 256, 0, st>>>(a);
  else if (pool && state) k_stream<T, OT, D, R, true, true><<<grid, 256, 0, st>>>(a);
  else if (pool) k_stream<T, OT, D, R, true, false><<<grid, 256, 0, st>>>(a);
  else if (rlds) k_stream<T, OT, D, R, false, true, true><<<grid, 256, 0, st>>>(a);
  else k_stream<T, OT, D, R, false, true><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <typename T, typename OT>
static hipError_t stream_by_shape(const Shape& s, const StreamArgs& a, bool pool, bool state, hipStream_t st) {
  if (!state) {  // pooling only: the rank does not matter
    return s.d == 64 ? stream_dispatch<T, OT, 64, 16>(s, a, pool, state, st)
                     : stream_dispatch<T, OT, 128, 16>(s, a, pool, state, st);
  }
  if (s.d == 64) {
    if (s.rank == 16) return stream_dispatch<T, OT, 64, 16>(s, a, pool, state, st);
    if (s.rank == 32) return stream_dispatch<T, OT, 64, 32>(s, a, pool, state, st);
    return stream_dispatch<T, OT, 64, 64>(s, a, pool, state, st);
  }
  if (s.rank == 16) return stream_dispatch<T, OT, 128, 16>(s, a, pool, state, st);
  if (s.rank == 32) return stream_dispatch<T, OT, 128, 32>(s, a, pool, state, st);
  return stream_dispatch<T, OT, 128, 64>(s, a, pool, state, st);
}

template <typename OT, int D, int R>
static hipError_t finalize_dispatch(const Shape& s, const FinalArgs& a, hipStream_t st) {
  k_finalize<OT, D, R><<<dim3(s.B * s.H, R / kFinRows), 256, 0, st>>>(a);
  return hipGetLastError();
}

template <typename OT>
static hipError_t finalize_by_shape(const Shape& s, const FinalArgs& a, hipStream_t st) {
  if (s.d == 64) {
    if (s.rank == 16) return finalize_dispatch<OT, 64, 16>(s, a, st);
    if (s.rank == 32) return finalize_dispatch<OT, 64, 32>(s, a, st);
    return finalize_dispatch<OT, 64, 64>(s, a, st);
  }
  if (s.rank == 16) return finalize_dispatch<OT, 128, 16>(s, a, st);
  if (s.rank == 32) return finalize_dispatch<OT, 128, 32>(s, a, st);
  return finalize_dispatch<OT, 128, 64>(s, a, st);
}

hipError_t launch_stream_f32(const Shape& s, const StreamArgs& a, bool pool, bool state, hipStream_t st);
hipError_t launch_finalize_f32(const Shape& s, const FinalArgs& a, hipStream_t st);

}  // namespace hsa
