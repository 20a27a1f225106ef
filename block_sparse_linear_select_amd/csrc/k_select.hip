// Tile selection: pooled score grid, per-row top-k and CSR emission.
//
// The sparse branch keeps only the high-energy query/key tile interactions
// (SparkDiffusion news article, section 05); at 90% / 97% sparsity that is 10% /
// 3% of the 64x64 tiles (same article, section 01), taken here as a fixed top-k
// per query-tile row.  Scores are float64 dot products of the float64 tile
// means, so the kept set is decided at the precision of the definition;
// ties are broken towards the lower tile index.
#include "common.hpp"
#include "kernels.hpp"

namespace hsa {

// -------------------------------------------------------------- keys
// Order-preserving 64-bit key of a float64 (larger key <=> larger value;
// -0 is folded onto +0 so that equal values tie).
__device__ __forceinline__ uint64_t order_key(double x) {
  if (x == 0.0) x = 0.0;
  uint64_t u = (uint64_t)__double_as_longlong(x);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}
// The same for a float32, in 32 bits.
__device__ __forceinline__ uint32_t order_key32(float x) {
  if (x == 0.f) x = 0.f;
  const uint32_t u = __float_as_uint(x);
  return (u >> 31) ? ~u : (u | 0x80000000u);
}

constexpr int kMaxJ = 32;  // up to 64 * 32 = 2048 tiles per row (keys per lane: MJ <= kMaxJ)

// The histogram of a radix pass is private to one wave, and the LDS
// operations of a wave complete in issue order: waiting for them and keeping
// the compiler from moving memory operations is all the ordering needed (a
// memory fence would also wait for the wave's outstanding global stores).
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
}

// Wave-wide reductions and scans on DPP lane moves within 16-lane rows plus
// four readlanes across the rows: no LDS traffic (a lane shuffle would go
// through the LDS crossbar and its latency).  Results are wave-uniform.
template <int CTRL>
__device__ __forceinline__ int dpp(int x) { return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xF, 0xF, false); }
template <int CTRL>
__device__ __forceinline__ float dppf(float x) { return __int_as_float(dpp<CTRL>(__float_as_int(x))); }
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kRowRor4 = 0x124, kRowRor8 = 0x128;

__device__ __forceinline__ int wave_max_int(int x) {
  x = max(x, dpp<kQuadXor1>(x));
  x = max(x, dpp<kQuadXor2>(x));
  x = max(x, dpp<kRowRor4>(x));
  x = max(x, dpp<kRowRor8>(x));
  const int a = max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16));
  const int b = max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48));
  return max(a, b);
}
__device__ __forceinline__ float wave_min_f(float x) {
  x = fminf(x, dppf<kQuadXor1>(x));
  x = fminf(x, dppf<kQuadXor2>(x));
  x = fminf(x, dppf<kRowRor4>(x));
  x = fminf(x, dppf<kRowRor8>(x));
  float r = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  r = fminf(r, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16)));
  r = fminf(r, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32)));
  return fminf(r, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48)));
}
// max over the 16 lanes of each row (every lane of the row gets it)
__device__ __forceinline__ float row16_max_f(float x) {
  x = fmaxf(x, dppf<kQuadXor1>(x));
  x = fmaxf(x, dppf<kQuadXor2>(x));
  x = fmaxf(x, dppf<kRowRor4>(x));
  return fmaxf(x, dppf<kRowRor8>(x));
}
// inclusive prefix sum over lanes 0..l (row scans by shifts, then the totals
// of the rows below)
__device__ __forceinline__ int wave_prefix_sum(int x, int lane) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane >> 4;
  return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}
// float64 sum over the wave: each row summed by lane moves of both halves,
// then the four row sums in a fixed order
__device__ __forceinline__ double dpp_d(double x, int ctrl_sel) {
  const int lo = __double2loint(x), hi = __double2hiint(x);
  int l2, h2;
  switch (ctrl_sel) {
    case 0: l2 = dpp<kQuadXor1>(lo); h2 = dpp<kQuadXor1>(hi); break;
    case 1: l2 = dpp<kQuadXor2>(lo); h2 = dpp<kQuadXor2>(hi); break;
    case 2: l2 = dpp<kRowRor4>(lo); h2 = dpp<kRowRor4>(hi); break;
    default: l2 = dpp<kRowRor8>(lo); h2 = dpp<kRowRor8>(hi); break;
  }
  return __hiloint2double(h2, l2);
}
__device__ __forceinline__ double readlane_d(double x, int l) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(x), l), __builtin_amdgcn_readlane(__double2loint(x), l));
}
__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
  for (int c = 0; c < 4; ++c) x += dpp_d(x, c);
  return ((readlane_d(x, 0) + readlane_d(x, 16)) + readlane_d(x, 32)) + readlane_d(x, 48);
}

__device__ __forceinline__ int wave_sum_int(int x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kRowRor4>(x);
  x += dpp<kRowRor8>(x);
  return (__builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16)) +
         (__builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48));
}

// The k-th largest of the values of the lanes in `live` (1 <= k <= their
// number, counting repeats), by ranking on the vector units: the 64 values go to
// a wave-private LDS buffer, every lane reads them all back (broadcast reads,
// 16 at a time) and counts those strictly above its own.  A value with fewer
// than k values above it is at least the k-th largest, and the k-th largest
// itself has fewer than k above it (ties included), so the k-th largest is the
// smallest such value: a wave minimum on lane moves, with the scalar unit
// (shared by the CU's waves) left free.
__device__ __forceinline__ float kth_largest_vec(float x, bool live, int k, int lane, float* buf) {
  const float xv = live ? x : -INFINITY;
  buf[lane] = xv;
  wave_lds_order();
  int gt = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    float4 o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = reinterpret_cast<const float4*>(buf)[4 * b + i];
#pragma unroll
    for (int i = 0; i < 4; ++i) gt += (o[i].x > xv) + (o[i].y > xv) + (o[i].z > xv) + (o[i].w > xv);
  }
  wave_lds_order();  // read before the buffer is written again
  return wave_min_f(live && gt < k ? xv : INFINITY);
}

// Top-k of one row held by one wave: key[j] of lane l belongs to column
// l + 64 j (j < nj); key 0 marks an absent column.  Radix select of the k-th
// largest key, 8 bits per pass; every key above it is kept and, among keys
// equal to it, the lowest columns.  Returns the kept flags (bit j of lane l:
// column l + 64 j).  `hw` is a 256-word LDS histogram owned by this wave.
template <int MJ, typename K>
__device__ uint32_t radix_topk(const K (&key)[MJ], int nj, int topk, int lane, uint32_t* hw) {
  constexpr int BITS = 8 * sizeof(K);
  // After each pass, `prefix` holds the bits fixed so far, `need` how many
  // keys of that bucket are still needed.  When a bucket holds exactly the
  // keys still needed, every key >= prefix is kept and the search stops
  // early (the usual case after two or three passes).
  K prefix = 0, mask = 0;
  int need = topk;
  bool done = false;
  // First pass (sign and top exponent bits): the keys of a row fall into a
  // handful of these digits, so LDS atomics would serialise.  Walk the
  // present digits from the top instead, counting each with ballots, and stop
  // at the digit that holds the k-th key.
  {
    uint32_t pend = 0;
#pragma unroll
    for (int j = 0; j < MJ; ++j)
      if (j < nj && key[j] != 0) pend |= 1u << j;
    int cum = 0, digit = 0, dcnt = 0;
    for (;;) {
      int dl = -1;
#pragma unroll
      for (int j = 0; j < MJ; ++j)
        if ((pend >> j) & 1u) dl = max(dl, (int)(key[j] >> (BITS - 8)));
      dl = wave_max_int(dl);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        if (j < nj) {
          const bool hit = ((pend >> j) & 1u) && (int)(key[j] >> (BITS - 8)) == dl;
          cnt += __popcll(__ballot(hit));
          if (hit) pend &= ~(1u << j);
        }
      }
      if (cum + cnt >= need || dl < 0) { digit = dl < 0 ? 0 : dl; dcnt = cnt; break; }
      cum += cnt;
    }
    need -= cum;
    prefix = (K)digit << (BITS - 8);
    mask = (K)255 << (BITS - 8);
    done = dcnt == need;
  }
  for (int shift = BITS - 16; shift >= 0 && !done; shift -= 8) {
    for (int i = lane; i < 256; i += 64) hw[i] = 0;
    wave_lds_order();
#pragma unroll
    for (int j = 0; j < MJ; ++j)
      if (j < nj && (key[j] & mask) == prefix && key[j] != 0)
        atomicAdd(&hw[(uint32_t)(key[j] >> shift) & 255u], 1u);
    wave_lds_order();
    // lane l owns digits 4l .. 4l+3; count from the top digit down
    const uint32_t h0 = hw[4 * lane], h1 = hw[4 * lane + 1], h2 = hw[4 * lane + 2], h3 = hw[4 * lane + 3];
    const uint32_t mine = h0 + h1 + h2 + h3;
    // count in the digits above this lane's (lanes above hold larger digits):
    // the total minus the inclusive prefix over lanes 0..l
    const int pre = wave_prefix_sum((int)mine, lane);
    const int tot = __builtin_amdgcn_readlane(pre, 63);
    uint32_t cum = (uint32_t)(tot - pre);
    int found = -1, rest = 0, fcnt = 0;
    const uint32_t hh[4] = {h0, h1, h2, h3};
#pragma unroll
    for (int dd = 3; dd >= 0; --dd) {
      if (found < 0 && cum < (uint32_t)need && cum + hh[dd] >= (uint32_t)need) {
        found = 4 * lane + dd;
        rest = need - (int)cum;
        fcnt = (int)hh[dd];
      }
      cum += hh[dd];
    }
    const uint64_t bal = __ballot(found >= 0);
    const int src_lane = bal ? __ffsll((unsigned long long)bal) - 1 : 0;
    const int digit = __builtin_amdgcn_readlane(found, src_lane);
    need = __builtin_amdgcn_readlane(rest, src_lane);
    const int bcnt = __builtin_amdgcn_readlane(fcnt, src_lane);
    prefix |= ((K)(digit < 0 ? 0 : digit)) << shift;
    mask |= (K)255 << shift;
    done = bcnt == need;
    wave_lds_order();
  }
  // keep key > kth, plus the `need` lowest-index keys equal to kth; an early
  // exit keeps every key >= prefix (kth = prefix - 1, no ties to break)
  const K kth = done ? prefix - 1 : prefix;
  if (done) need = 0;
  uint32_t sel = 0;
  int taken = 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int j = 0; j < MJ; ++j) {
    if (j < nj) {  // nj is wave-uniform; a guard instead of a break keeps key[] in registers
      const bool above = key[j] > kth;
      const bool eq = key[j] == kth && key[j] != 0;
      const uint64_t be = __ballot(eq);
      const int before = __popcll(be & lt_mask);
      if (above || (eq && taken + before < need)) sel |= 1u << j;
      taken += __popcll(be);
    }
  }
  return sel;
}

// -------------------------------------------------------------- selection
// One block = 16 consecutive query tiles of one (b, h), four waves.
//
//  1. Pooling: float64 sums of the valid rows of each query tile (exact for
//     bf16 and fp8 values), divided by the valid count -> qbar (written to
//     the workspace and, if asked, exported).
//  2. Scores: sigma'_ab = qbar_a . kbar_b for every key tile b on the bf16
//     matrix cores, each float64 mean split into bf16 hi + lo parts and the
//     three products hi.hi + hi.lo + lo.hi accumulated in float32.  A fourth
//     product |qbar_hi| . |kbar_hi| gives A_ab >= sum_e |qbar_e kbar_e| / (1 + 2^-7)^2,
//     and |sigma' - sigma| <= 1.6e-4 A_ab bounds the error (dropped lo.lo
//     and remainder terms: 3.05 * 2^-16; 384 float32 additions: 2.3e-5;
//     a factor 2.2 of margin).
//  3. Top-k: per row, the approximate top-k A' by (sigma' desc, b asc) and
//     t' = its smallest score.  With E = the row's largest error bound,
//     every tile with sigma' > t' + 2E is in the exact top-k, every tile with
//     sigma' < t' - 2E is out, and only the tiles in between are ranked again
//     by their exact float64 scores (usually none: the band is ~1e-4 of the
//     scores, the gap at the k-th score ~1e-3).  So the kept set is exactly
//     the one the float64 scores give, ties to the lower index.
//  4. Emission: the kept tiles in ascending order (plus the diagonal when
//     forced) as a CSR row.
struct SelectArgs {
  int T, N, N_pad, topk, force_diag, direct;
  const void* q;        // [BH][N_pad][D] in the input type
  const float* qs;      // fp8: [BH][T] tile scales of Q
  const uint16_t* khi;  // bf16 hi part of the key tile means, fragment order (kfrag_index)
  const uint16_t* klo;  // bf16 lo part, the same order
  const double* kmean;  // [BH][T][D]
  double* qmean;        // [BH][T][D], written
  double* qbar_out;     // optional export [BH][T][D]
  int32_t* out_cols;    // direct: col_idx [rows][topk]; else [rows][topk + 1]
  int32_t* out_cnt;     // [rows] when not direct
  int32_t* row_ptr;     // [rows + 1] when direct
  int rows;
  int nbh;              // B * H
};

constexpr int kSelRows = 16;  // query tiles per block
constexpr float kScoreErr = 1.6e-4f;

// float64 -> bf16 bits (through float32; the bound above allows the double rounding)
__device__ __forceinline__ uint32_t bf16_of(double x) { return f32_to_bf16_bits((float)x); }
__device__ __forceinline__ double bf16_value(uint32_t b) { return (double)bf16_bits_to_f32(b); }

template <typename IT, int D, int MJ>
__global__ __launch_bounds__(256, 2) void k_select(SelectArgs a) {
  constexpr int CPR = D / 8, NCONT = 256 / CPR, KCH = 64 * CPR / 256;
  constexpr int TP = 64 * MJ + 4;           // row stride of the scores (+4 words: rows on distinct banks)
  constexpr int POOL_BYTES = NCONT * D * 8;  // pooling partials (float64)
  constexpr int QF_BYTES = 2 * kSelRows * D * 2;
  constexpr int SC_BYTES = kSelRows * TP * 4;
  constexpr int SMEM = (2 * POOL_BYTES + QF_BYTES > SC_BYTES) ? 2 * POOL_BYTES + QF_BYTES : SC_BYTES;
  constexpr bool SCALED = sizeof(IT) == 1;
  __shared__ __align__(16) uint8_t smem[SMEM];
  __shared__ float emax[4][kSelRows];
  double* red = reinterpret_cast<double*>(smem);
  uint16_t* qh = reinterpret_cast<uint16_t*>(smem + 2 * POOL_BYTES);  // [16][D]
  uint16_t* ql = qh + kSelRows * D;
  float* sc = reinterpret_cast<float*>(smem);  // [16][TP], once the pooling is done

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int T = a.T;
  // Block order: the hardware hands block i to XCD i % 8.  XCD x takes heads
  // x, x + 8, ... one after the other, so the head whose key means its blocks
  // read (kept in its L2) is shared by all of its blocks in flight.
  const int nrb = (T + kSelRows - 1) / kSelRows;
  const int xcd = blockIdx.x & 7, jb = blockIdx.x >> 3;
  const int bh = xcd + 8 * (jb / nrb), a0 = (jb % nrb) * kSelRows;
  if (bh >= a.nbh) return;
  const int nr = min(kSelRows, T - a0);
  const size_t tb = (size_t)bh * T;

  // ---- 1. pooling of the block's query tiles (four tiles of loads in flight, two reduced per round)
  {
    const IT* Q = reinterpret_cast<const IT*>(a.q) + (size_t)bh * a.N_pad * D;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q, a.N * D * (int)sizeof(IT));
    const int col8 = tid % CPR, row0 = tid / CPR;
    Chunk8<IT> cq[4][KCH];
    auto load = [&](int r, int slot) {
      // a tile past the block's range reads beyond the view: zeros, no traffic
      const int t = r < nr ? a0 + r : T;
#pragma unroll
      for (int i = 0; i < KCH; ++i) bload8(cq[slot][i], qrs, (t * 64 + row0 + i * NCONT) * D + col8 * 8);
    };
    // partial column sums of the tile in register slot `slot` into partial
    // region h; the slot then loads the tile four ahead
    auto partials = [&](int r, int slot, int h) {
      double p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = 0.0;
#pragma unroll
      for (int i = 0; i < KCH; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] += (double)elem(cq[slot][i], e);
      load(r + 4, slot);  // the registers are free again: the tile four ahead
#pragma unroll
      for (int e = 0; e < 8; ++e) red[h * NCONT * D + row0 * D + col8 * 8 + e] = p[e];
    };
    // two tiles per round (r and r + 1, slots s0 and s0 + 1): one barrier
    // publishes both tiles' partials, and threads tid < 2 D finish the means
    // of both, column tid % D of tile r + tid / D
    auto reduce2 = [&](int r, int s0) {
      partials(r, s0, 0);
      if (r + 1 < nr) partials(r + 1, s0 + 1, 1);
      __syncthreads();
      const int h = tid / D, col = tid % D;
      if (h < 2 && r + h < nr) {
        const int at = a0 + r + h;
        const double* rh = red + h * NCONT * D;
        double sum = 0.0;
#pragma unroll 4
        for (int c2 = 0; c2 < NCONT; ++c2) sum += rh[c2 * D + col];
        if constexpr (SCALED) sum *= (double)a.qs[tb + at];
        const int cnt = min(64, a.N - at * 64);  // a full tile: exactly a multiply by 2^-6
        const double mean = cnt == 64 ? sum * 0.015625 : sum / (double)cnt;
        const size_t o = (tb + at) * D + col;
        a.qmean[o] = mean;
        if (a.qbar_out) a.qbar_out[o] = mean;
        const uint32_t hb = bf16_of(mean);
        qh[(r + h) * D + col] = (uint16_t)hb;
        ql[(r + h) * D + col] = (uint16_t)bf16_of(mean - bf16_value(hb));
      }
      __syncthreads();
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) load(i, i);
    for (int r = 0; r < nr; r += 4) {
      reduce2(r, 0);
      if (r + 2 < nr) reduce2(r + 2, 2);
    }
    for (int i = tid; i < (kSelRows - nr) * D; i += 256) {  // rows past T: zero operands
      qh[nr * D + i] = 0;
      ql[nr * D + i] = 0;
    }
  }
  __syncthreads();

  // ---- 2. approximate scores and their error bounds
  Frag<bf16_t> ah[D / 32], al[D / 32], aa[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    ah[c].w = *reinterpret_cast<const u32x4*>(&qh[l16 * D + 32 * c + 8 * g]);
    al[c].w = *reinterpret_cast<const u32x4*>(&ql[l16 * D + 32 * c + 8 * g]);
#pragma unroll
    for (int i = 0; i < 4; ++i) aa[c].w[i] = ah[c].w[i] & 0x7FFF7FFFu;
  }
  __syncthreads();  // the operands are in registers: the region now holds scores
  // the head's key means in fragment order as bounds-checked buffers: the
  // padding of the last key block holds zeros, blocks past it read as zeros
  const size_t kfb = (size_t)bh * kfrag_tiles(T) * D;
  const __amdgpu_buffer_rsrc_t khr = make_rsrc(a.khi + kfb, kfrag_tiles(T) * D * 2);
  const __amdgpu_buffer_rsrc_t klr = make_rsrc(a.klo + kfb, kfrag_tiles(T) * D * 2);
  const int nkb = (T + 15) / 16;
  float em[4] = {0.f, 0.f, 0.f, 0.f};
  // three key blocks of operands in flight per wave (blocks w, w + 4, w + 8, ...)
  Frag<bf16_t> bhf[3][D / 32], blf[3][D / 32];
  auto loadb = [&](int kb, int slot) {
    const int off = (kb * (D / 32) * 64 + lane) * 16;  // one 1 KB run per (kb, c)
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      bhf[slot][c].w = __builtin_amdgcn_raw_buffer_load_b128(khr, off + 1024 * c, 0, 0);
      blf[slot][c].w = __builtin_amdgcn_raw_buffer_load_b128(klr, off + 1024 * c, 0, 0);
    }
  };
  auto scores = [&](int kb, int slot) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acca = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      Frag<bf16_t> babs;
#pragma unroll
      for (int i = 0; i < 4; ++i) babs.w[i] = bhf[slot][c].w[i] & 0x7FFF7FFFu;
      mma(acc, ah[c], bhf[slot][c]);
      mma(acc, ah[c], blf[slot][c]);
      mma(acc, al[c], bhf[slot][c]);
      mma(acca, aa[c], babs);
    }
    loadb(kb + 12, slot);  // in flight while the next two blocks are multiplied
    // accumulator: lane holds column b = 16 kb + l16, rows 4 g + i
    const int b = 16 * kb + l16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[(4 * g + i) * TP + b] = acc[i];
      em[i] = fmaxf(em[i], acca[i]);
    }
  };
  loadb(w, 0);
  loadb(w + 4, 1);
  loadb(w + 8, 2);
  for (int kb = w; kb < nkb; kb += 12) {
    scores(kb, 0);
    if (kb + 4 < nkb) scores(kb + 4, 1);
    if (kb + 8 < nkb) scores(kb + 8, 2);
  }
  // largest bound per row: over the 16 columns of a lane group, then the waves
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    em[i] = row16_max_f(em[i]);
    if (l16 == 0) emax[w][4 * g + i] = em[i];
  }
  __syncthreads();

  // ---- 3. top-k of each row and 4. emission (wave w: rows w, w + 4, ...)
  const int nj = (T + 63) / 64;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int kept[kSelRows / 4] = {0, 0, 0, 0};
  // bit j: column lane + 64 j exists (columns past T read the row's padding)
  uint32_t vmask = 0;
#pragma unroll
  for (int j = 0; j < MJ; ++j) vmask |= (lane + 64 * j < T ? 1u : 0u) << j;
  for (int r = w; r < nr; r += 4) {
    const int at = a0 + r;
    const int row = (int)(tb + at);
    float sv[MJ];
#pragma unroll
    for (int j = 0; j < MJ; ++j) sv[j] = sc[r * TP + lane + 64 * j];
    auto ok = [&](int j) { return ((vmask >> j) & 1u) != 0u; };
    // this row's part of the score region now serves as scratch of this wave
    uint32_t* hw = reinterpret_cast<uint32_t*>(&sc[r * TP]);
    float* slot = &sc[r * TP];
    wave_lds_order();
    const int k = min(a.topk, T);
    // t' = the k-th largest approximate score (counting repeats).  The k-th
    // largest of the 64 lane maxima is a lower bound theta of t' (k of them
    // are at least theta), so the top-k lies among the scores >= theta; when
    // those are at most 64 (the usual case), t' is found by ranking them one
    // per lane.  Otherwise, a radix select over all scores.
    float tmin = 0.f;
    bool fast = false;
    if (k <= 64) {
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < MJ; ++j)
        if (ok(j)) mx = fmaxf(mx, sv[j]);
      const float theta = kth_largest_vec(mx, mx > -INFINITY, k, lane, slot + 64);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < MJ; ++j) cnt += (ok(j) && sv[j] >= theta) ? 1 : 0;
      const int pre = wave_prefix_sum(cnt, lane);
      const int c = __builtin_amdgcn_readlane(pre, 63);
      if (c <= 64) {
        int pos = pre - cnt;  // this lane's candidates go to slots pos, pos + 1, ...
#pragma unroll
        for (int j = 0; j < MJ; ++j) {
          if (ok(j) && sv[j] >= theta) slot[pos++] = sv[j];
        }
        wave_lds_order();
        const float cv = lane < c ? slot[lane] : -INFINITY;
        tmin = kth_largest_vec(cv, lane < c, k, lane, slot + 64);
        fast = true;
        wave_lds_order();  // the slots are read before the region is used again
      }
    }
    if (!fast) {
      uint32_t key[MJ];  // order-preserving keys, 0 for absent columns
#pragma unroll
      for (int j = 0; j < MJ; ++j) key[j] = ok(j) ? order_key32(sv[j]) : 0u;
      const uint32_t sel = radix_topk<MJ>(key, nj, k, lane, hw);
      tmin = INFINITY;
#pragma unroll
      for (int j = 0; j < MJ; ++j)
        if ((sel >> j) & 1u) tmin = fminf(tmin, sv[j]);
      tmin = wave_min_f(tmin);
    }
    uint32_t sel = 0;
    const float E = kScoreErr * fmaxf(fmaxf(emax[0][r], emax[1][r]), fmaxf(emax[2][r], emax[3][r]));
    const float hi = tmin + 2.f * E, lo = tmin - 2.f * E;
    uint32_t fin = 0, fcand = 0;
    int cin = 0, ccand = 0;
#pragma unroll
    for (int j = 0; j < MJ; ++j) {
      const bool in = ok(j) && sv[j] > hi;
      const bool cand = ok(j) && !in && sv[j] >= lo;
      fin |= (in ? 1u : 0u) << j;
      fcand |= (cand ? 1u : 0u) << j;
      cin += in ? 1 : 0;
      ccand += cand ? 1 : 0;
    }
    const int nin = wave_sum_int(cin), ncand = wave_sum_int(ccand);
    if (ncand != k - nin) {
      // rank the candidates by their exact float64 scores: in-tiles get the
      // largest key, candidates order_key(sigma), the rest stay absent.  A few
      // candidates: one wave-wide dot product each; many (degenerate rows,
      // e.g. an all-zero query tile, where every score ties): one per lane.
      const double* qrow = a.qmean + (tb + at) * D;  // written by this block before a barrier
      const bool few = ncand <= 4;
      uint64_t key64[MJ];
      double qv[D / 64];
#pragma unroll
      for (int e = 0; e < D / 64; ++e) qv[e] = qrow[lane + 64 * e];
#pragma unroll
      for (int j = 0; j < MJ; ++j) key64[j] = ((fin >> j) & 1u) ? ~0ull : 0ull;
      if (few) {
        // the (at most four) candidate columns, their key means loaded together
        int cidx[4] = {0, 0, 0, 0};
        int n = 0;
#pragma unroll
        for (int j = 0; j < MJ; ++j) {
          if (j < nj) {
            uint64_t bal = __ballot((fcand >> j) & 1u);
            while (bal) {
              const int src = __ffsll((unsigned long long)bal) - 1;
              bal &= bal - 1;
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (i == n) cidx[i] = src + 64 * j;
              ++n;
            }
          }
        }
        double kv[4][D / 64];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < D / 64; ++e)
            kv[i][e] = i < n ? a.kmean[(tb + cidx[i]) * D + lane + 64 * e] : 0.0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i < n) {
            double part = 0.0;
#pragma unroll
            for (int e = 0; e < D / 64; ++e) part = fma(qv[e], kv[i][e], part);
            part = wave_sum_d(part);
            const int b = cidx[i];
#pragma unroll
            for (int j = 0; j < MJ; ++j)
              if (lane + 64 * j == b) key64[j] = order_key(part);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < MJ; ++j) {
          if (j < nj && ((fcand >> j) & 1u)) {
            const double2* krow = reinterpret_cast<const double2*>(a.kmean + (tb + lane + 64 * j) * D);
            const double2* qr2 = reinterpret_cast<const double2*>(qrow);
            double acc = 0.0;
#pragma unroll 4
            for (int e = 0; e < D / 2; ++e) {
              const double2 kk = krow[e], qq = qr2[e];
              acc = fma(qq.x, kk.x, acc);
              acc = fma(qq.y, kk.y, acc);
            }
            key64[j] = order_key(acc);
          }
        }
      }
      wave_lds_order();
      sel = radix_topk<MJ>(key64, nj, k, lane, hw);
    } else {
      sel = fin | fcand;
    }
    if (a.force_diag && lane == (at & 63)) sel |= 1u << (at >> 6);

    // emit ascending: the kept columns are gathered in LDS, then stored contiguously
    int base_pos = 0;
    int* oslot = reinterpret_cast<int*>(slot);
    wave_lds_order();
#pragma unroll
    for (int j = 0; j < MJ; ++j) {
      if (j < nj) {
        const bool s = (sel >> j) & 1u;
        const uint64_t bs = __ballot(s);
        if (s) oslot[base_pos + __popcll(bs & lt_mask)] = lane + 64 * j;
        base_pos += __popcll(bs);
      }
    }
    // the list stays in LDS: the wave stores its rows' lists after its last
    // row, so that no load of the loop waits behind these stores
    kept[(r - w) >> 2] = base_pos;
    if (lane == 0) {
      if (a.direct) {
        a.row_ptr[row] = row * a.topk;
        if (row == a.rows - 1) a.row_ptr[a.rows] = a.rows * a.topk;
      } else {
        a.out_cnt[row] = base_pos;
      }
    }
  }
  wave_lds_order();
#pragma unroll
  for (int q = 0; q < kSelRows / 4; ++q) {
    const int r = w + 4 * q;
    if (r < nr) {
      const int row = (int)(tb + a0 + r);
      const size_t obase = a.direct ? (size_t)row * a.topk : (size_t)row * (a.topk + 1);
      const int* oslot = reinterpret_cast<const int*>(&sc[r * TP]);
      for (int i = lane; i < kept[q]; i += 64) a.out_cols[obase + i] = oslot[i];
    }
  }
}

// Exclusive scan of the per-row counts into row_ptr (single block).
__global__ __launch_bounds__(1024) void k_scan(int rows, const int32_t* __restrict__ cnt, int32_t* __restrict__ row_ptr) {
  __shared__ int32_t part[1024];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < rows; base += 1024) {
    int i = base + threadIdx.x;
    int v = i < rows ? cnt[i] : 0;
    part[threadIdx.x] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      int t = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
      __syncthreads();
      part[threadIdx.x] += t;
      __syncthreads();
    }
    if (i < rows) row_ptr[i] = carry + part[threadIdx.x] - v;
    __syncthreads();
    if (threadIdx.x == 1023) carry += part[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) row_ptr[rows] = carry;
}

__global__ void k_compact(int rows, int stride, const int32_t* __restrict__ tmp, const int32_t* __restrict__ cnt,
                          const int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx) {
  int row = blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= rows) return;
  int n = cnt[row], o = row_ptr[row];
  for (int i = 0; i < n; ++i) col_idx[o + i] = tmp[(size_t)row * stride + i];
}

template <typename IT, int D>
static void select_by_mj(int nj, dim3 grid, const SelectArgs& a, hipStream_t st) {
  if (nj <= 8) k_select<IT, D, 8><<<grid, 256, 0, st>>>(a);
  else if (nj <= 16) k_select<IT, D, 16><<<grid, 256, 0, st>>>(a);
  else if (nj <= 19) k_select<IT, D, 19><<<grid, 256, 0, st>>>(a);
  else if (nj <= 24) k_select<IT, D, 24><<<grid, 256, 0, st>>>(a);
  else k_select<IT, D, kMaxJ><<<grid, 256, 0, st>>>(a);
}

hipError_t launch_select(const Shape& s, const void* q, const float* qs, const Scratch& w, int32_t* row_ptr,
                         int32_t* col_idx, double* qbar_out, hipStream_t st) {
  const int rows = s.B * s.H * s.T;
  const int direct = s.force_diag ? 0 : 1;
  SelectArgs a{};
  a.T = s.T; a.N = s.N; a.N_pad = s.N_pad; a.topk = s.topk; a.force_diag = s.force_diag; a.direct = direct;
  a.q = q; a.qs = qs; a.khi = w.khi; a.klo = w.klo; a.kmean = w.kmean; a.qmean = w.qmean; a.qbar_out = qbar_out;
  a.out_cols = direct ? col_idx : w.sel_tmp;
  a.out_cnt = w.sel_cnt;
  a.row_ptr = row_ptr;
  a.rows = rows;
  a.nbh = s.B * s.H;
  const int nj = (s.T + 63) / 64;
  const dim3 grid(8 * ((s.B * s.H + 7) / 8) * ((s.T + kSelRows - 1) / kSelRows));
  if (s.d == 64) {
    if (s.dt == Dt::F32) select_by_mj<float, 64>(nj, grid, a, st);
    else if (s.dt == Dt::BF16) select_by_mj<bf16_t, 64>(nj, grid, a, st);
    else select_by_mj<fp8_t, 64>(nj, grid, a, st);
  } else {
    if (s.dt == Dt::F32) select_by_mj<float, 128>(nj, grid, a, st);
    else if (s.dt == Dt::BF16) select_by_mj<bf16_t, 128>(nj, grid, a, st);
    else select_by_mj<fp8_t, 128>(nj, grid, a, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || direct) return e;
  k_scan<<<1, 1024, 0, st>>>(rows, w.sel_cnt, row_ptr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_compact<<<(rows + 255) / 256, 256, 0, st>>>(rows, s.topk + 1, w.sel_tmp, w.sel_cnt, row_ptr, col_idx);
  return hipGetLastError();
}

}  // namespace hsa
