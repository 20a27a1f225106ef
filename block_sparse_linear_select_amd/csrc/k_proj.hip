// W8A8 FP8 QKV projection in front of the attention (SparkDiffusion news
// article, section 07: the linear projections run as W8A8 FP8 E4M3 with the
// activation scaling and the type conversions fused into the kernels; the
// project blog, "A simple staging principle", item 3).
//
//  * k_quant_rows: per-token-row E4M3 quantisation of bf16 activations,
//    s_x = max|x| / 448, code = round-to-nearest-even(x / s_x).  One wave per
//    row, two passes over the row (the second from L2).
//  * k_proj_fp8: Y = diag(s_x) X8 W8^T diag(s_w) on the fp8 matrix cores, with
//    the output quantisation of the attention's FP8 input fused into the
//    epilogue: each block owns 256 tokens (four 64-token tiles) x 256 output
//    columns (two heads), so every per-(tile, head) scale is decided inside
//    one block, and the codes are written straight into the [B, H, N_pad, d]
//    layout the attention reads.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_dma.hpp"

namespace hsa {

// --------------------------------------------------------- activation rows
// x: bf16 [M, C], C a multiple of 8.  Exact: max|x| is exact, and both
// divisions are correctly rounded float32 divisions.
__global__ __launch_bounds__(256) void k_quant_rows(const uint16_t* __restrict__ x, long M, int C,
                                                   uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const long m = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  const uint16_t* row = x + (size_t)m * C;
  const int nch = C / 8;  // 16-byte chunks of the row
  float amax = 0.f;
  for (int c = lane; c < nch; c += 64) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(row + 8 * c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[j] & 0xFFFFu)));
      amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[j] >> 16)));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const float s = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
  uint8_t* out = codes + (size_t)m * C;
  for (int c = lane; c < nch; c += 64) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(row + 8 * c);
    uint32_t w2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float y0 = __fdiv_rn(bf16_bits_to_f32(v[2 * h] & 0xFFFFu), s);
      const float y1 = __fdiv_rn(bf16_bits_to_f32(v[2 * h] >> 16), s);
      const float y2 = __fdiv_rn(bf16_bits_to_f32(v[2 * h + 1] & 0xFFFFu), s);
      const float y3 = __fdiv_rn(bf16_bits_to_f32(v[2 * h + 1] >> 16), s);
      int p = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
      w2[h] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, p, true);
    }
    *reinterpret_cast<uint2*>(out + 8 * c) = make_uint2(w2[0], w2[1]);
  }
  if (lane == 0) scales[m] = s;
}

// ------------------------------------------------------------- projection
struct ProjArgs {
  const uint8_t* x;  // [M, C] E4M3 codes of the activations (M = B * N_pad)
  const float* sx;   // [M]
  const uint8_t* w;  // [3 H d, C] E4M3 codes of the weights
  const float* sw;   // [3 H d]
  uint8_t* out[3];   // q, k, v codes [B, H, N_pad, d]
  float* osc[3];     // their scales [B, H, T]
  long M;
  int C, H, n_pad, T;
};

constexpr int kPM = 256;   // tokens per block (four 64-token tiles)
constexpr int kPN = 256;   // output columns per block (two heads, d = 128)
constexpr int kPK = 128;   // contraction bytes per stage (one 16x16x128 step)
constexpr int kPWaves = 8; // 2 token halves x 4 column quarters
constexpr int kPXL = kPM * kPK / 1024 / kPWaves;  // LDS-direct loads per wave per stage: activations
constexpr int kPWL = kPN * kPK / 1024 / kPWaves;  // ... and weights
constexpr int kPLoads = kPXL + kPWL;

// Tile rows are 128 bytes (8 granules); granule p of row r sits at position
// p ^ f(r), f(r) = 2 (r mod 4) + bit 2 of r.  On gfx950 this swizzle reads
// with no LDS bank conflicts (measured by the bank-conflict counter over
// every XOR swizzle linear in the row bits; r & 7 and (r >> 1) & 7 cost 4
// conflict cycles per 16-byte read instruction).
__device__ __forceinline__ int swz_p(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

// Block: 8 waves; wave (wr, wc) computes tokens 128 wr .. +127 x columns
// 64 wc .. +63 as 4 x 8 steps of 16 columns x 16 tokens: A = W rows (columns
// of Y), B = X rows (tokens), so a lane's accumulator holds 4 consecutive
// columns of one token, written as one 4-byte store.  A wave tile of 128 x 64
// reads 24 KB of LDS per stage for 32 steps.  Two LDS stages: the loads of
// stage s + 1 are issued at the start of stage s and have its 32 steps per
// wave (two waves per SIMD) to land.
__global__ __launch_bounds__(64 * kPWaves, 1) void k_proj_fp8(ProjArgs a) {
  __shared__ __align__(16) uint8_t Ws[2][kPN * kPK];
  __shared__ __align__(16) uint8_t Xs[2][kPM * kPK];
  __shared__ float amax_sh[4][4];  // [64-token tile][column quarter]

  const int ncb = (3 * a.H + 1) / 2;  // 256-column blocks (the last may hold one head)
  const int cb = uniform(blockIdx.x % ncb);
  const long m0 = (long)uniform(blockIdx.x / ncb) * kPM;
  const int j0 = cb * kPN;
  const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
  const int wr = w >> 2, wc = w & 3, l16 = lane & 15, g = lane >> 4;

  // This block's 256 weight rows and 256 activation rows; rows past the end
  // (M, or 3 H d for a last block of one head) read as zeros through the
  // bounds-checked views.
  const long mrows = min((long)kPM, a.M - m0);
  const int wrows = min(kPN, 3 * a.H * 128 - j0);
  const i32x4_t wrs = make_rsrc_regs(a.w + (size_t)j0 * a.C, wrows * a.C);
  const i32x4_t xrs = make_rsrc_regs(a.x + (size_t)m0 * a.C, (int)mrows * a.C);
  // LDS-direct load i of a tile fills bytes [1024 i, +1024): rows 8 i + lane / 8,
  // slot lane % 8; the slot holds granule slot ^ swz(row).  The lane part of
  // the source offset depends on i only through i & 1 (with rows 8 i + lane / 8
  // and a swizzle of r mod 8, not at all).
  int lp[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = 8 * r + lane / 8;
    lp[r] = (lane / 8) * a.C + 16 * ((lane % 8) ^ swz_p(row));
  }
  auto stage = [&](int s, int buf) {
    const int k0 = s * kPK;
    static_for<0, kPXL>([&](auto ic) {
      constexpr int ii = decltype(ic)::value;
      const int i = kPXL * w + ii;
      lds_dma16<1024 * ii>(xrs, &Xs[buf][1024 * kPXL * w], lp[i & 1] + 8 * i * a.C + k0);
    });
    static_for<0, kPWL>([&](auto ic) {
      constexpr int ii = decltype(ic)::value;
      const int i = kPWL * w + ii;
      lds_dma16<1024 * ii>(wrs, &Ws[buf][1024 * kPWL * w], lp[i & 1] + 8 * i * a.C + k0);
    });
  };
  if (a.C < 0) { Ws[0][tid] = 0; Xs[0][tid] = 0; }  // never executed: the tiles are written by LDS-direct loads

  f32x4 acc[4][8];
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int tb = 0; tb < 8; ++tb) acc[fb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment (row of the tile, bytes 32 g .. +31): granules 2g, 2g + 1
  auto frag = [&](const uint8_t* tile, int row) {
    const int sw = swz_p(row);
    const u32x4 lo = *reinterpret_cast<const u32x4*>(tile + row * kPK + 16 * ((2 * g) ^ sw));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(tile + row * kPK + 16 * ((2 * g + 1) ^ sw));
    return cat8(lo, hi);
  };

  const int nk = a.C / kPK;
  stage(0, 0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  lds_barrier();
  for (int s = 0; s < nk; ++s) {
    const int cur = s & 1;
    if (s + 1 < nk) stage(s + 1, cur ^ 1);  // lands while this stage's steps run
    i32x8_t af[4];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) af[fb] = frag(Ws[cur], 64 * wc + 16 * fb + l16);
#pragma unroll
    for (int tb = 0; tb < 8; ++tb) {
      const i32x8_t bf = frag(Xs[cur], 128 * wr + 16 * tb + l16);
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) acc[fb][tb] = mma_fp8(af[fb], bf, acc[fb][tb]);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // this wave's share of the next stage has landed
    lds_barrier();                              // next stage visible; every wave is done with this one
  }

  // ---- epilogue: scale, per-(tile, head) absmax, E4M3 codes
  float swv[4][4];
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + 64 * wc + 16 * fb + 4 * g + i;
      swv[fb][i] = j < 3 * a.H * 128 ? a.sw[j] : 0.f;
    }
  float amax[2] = {0.f, 0.f};  // this wave's two 64-token tiles
#pragma unroll
  for (int tb = 0; tb < 8; ++tb) {
    const long m = m0 + 128 * wr + 16 * tb + l16;
    const float sx = m < a.M ? a.sx[m] : 0.f;
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float y = acc[fb][tb][i] * sx * swv[fb][i];
        acc[fb][tb][i] = y;
        amax[tb >> 2] = fmaxf(amax[tb >> 2], fabsf(y));
      }
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax[q] = fmaxf(amax[q], __shfl_xor(amax[q], off, 64));
    if (lane == 0) amax_sh[2 * wr + q][wc] = amax[q];
  }
  __syncthreads();
  const int t_unit = 2 * cb + (wc >> 1);  // the head unit of this wave's columns
  if (t_unit >= 3 * a.H) return;
  const int t = t_unit / a.H, h = t_unit % a.H;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const long mh = m0 + 128 * wr + 64 * q;  // first token of the tile
    if (mh >= a.M) break;
    const float am = fmaxf(amax_sh[2 * wr + q][wc & 2], amax_sh[2 * wr + q][(wc & 2) + 1]);
    const float sc = am > 0.f ? __fdiv_rn(am, 448.f) : 1.f;
    const float inv = __fdiv_rn(1.f, sc);
    const long b = mh / a.n_pad;
    const int n0 = (int)(mh - b * a.n_pad);
    uint8_t* dst = a.out[t] + (((size_t)b * a.H + h) * a.n_pad + n0) * 128 + 64 * (wc & 1) + 4 * g;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        const f32x4 y = acc[fb][4 * q + tt];
        int p = __builtin_amdgcn_cvt_pk_fp8_f32(y[0] * inv, y[1] * inv, 0, false);
        p = __builtin_amdgcn_cvt_pk_fp8_f32(y[2] * inv, y[3] * inv, p, true);
        *reinterpret_cast<uint32_t*>(dst + (size_t)(16 * tt + l16) * 128 + 16 * fb) = (uint32_t)p;
      }
    if ((wc & 1) == 0 && lane == 0) a.osc[t][((size_t)b * a.H + h) * a.T + n0 / 64] = sc;
  }
}

hipError_t launch_quant_rows(const void* x, long M, int C, void* codes, float* scales, hipStream_t st) {
  if (M == 0) return hipSuccess;
  const long grid = (M + 3) / 4;
  k_quant_rows<<<dim3((unsigned)grid), 256, 0, st>>>(static_cast<const uint16_t*>(x), M, C,
                                                      static_cast<uint8_t*>(codes), scales);
  return hipGetLastError();
}

hipError_t launch_proj_fp8(const void* x, const float* sx, const void* wq, const float* sw, long M, int C, int H,
                           int n_pad, void* const* out, float* const* osc, hipStream_t st) {
  if (M == 0) return hipSuccess;
  ProjArgs a{};
  a.x = static_cast<const uint8_t*>(x);
  a.sx = sx;
  a.w = static_cast<const uint8_t*>(wq);
  a.sw = sw;
  for (int t = 0; t < 3; ++t) { a.out[t] = static_cast<uint8_t*>(out[t]); a.osc[t] = osc[t]; }
  a.M = M; a.C = C; a.H = H; a.n_pad = n_pad; a.T = n_pad / 64;
  const long grid = ((M + kPM - 1) / kPM) * ((3 * H + 1) / 2);
  k_proj_fp8<<<dim3((unsigned)grid), 64 * kPWaves, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace hsa
