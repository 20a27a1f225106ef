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

// -------------------------------------------------------------- scores
// sigma[a][b] = qbar_a . kbar_b for one (b, h), float64 16x16x4 matrix-core
// steps.  Block: 4 waves x 16 rows = 64 rows of a; the column means are
// staged 32 columns at a time through double-buffered LDS, and each wave runs
// two independent accumulator chains.  Means are stored one row per tile
// ([T][d]): a chunk of 32 column means is one contiguous block, loaded
// coalesced and kept in LDS with row stride d + 4 doubles (the 16 rows x 4
// dims of an operand read then spread over all banks).
constexpr int kScoreCols = 32;

template <int D>
__global__ __launch_bounds__(256) void k_scores(int T, const double* __restrict__ qmean,
                                                const double* __restrict__ kmean, double* __restrict__ scores) {
  constexpr int CS = D + 4;  // LDS row stride (doubles) of a staged column mean
  __shared__ double kbuf[2][kScoreCols * CS];
  const int bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const double* qb = qmean + (size_t)bh * T * D;
  const double* kb = kmean + (size_t)bh * T * D;
  double* out = scores + (size_t)bh * T * T;
  const int rbase = 64 * blockIdx.x + 16 * w;
  const int row = rbase + l16;
  double af[D / 4];
#pragma unroll
  for (int s = 0; s < D / 4; ++s) af[s] = row < T ? qb[(size_t)row * D + 4 * s + g] : 0.0;

  // this block's part of the columns: chunks [c_lo, c_hi) of blockIdx.z's share
  const int nchunks_all = (T + kScoreCols - 1) / kScoreCols;
  const int c_lo = (int)((long)nchunks_all * blockIdx.z / gridDim.z);
  const int c_hi = (int)((long)nchunks_all * (blockIdx.z + 1) / gridDim.z);
  // each thread stages PER doubles of a chunk: element tid + 256 i of the
  // chunk's contiguous [32][D] block
  constexpr int PER = D * kScoreCols / 256;
  double pre[PER];
  auto fetch = [&](int cc) {
    const double* src = kb + (size_t)cc * kScoreCols * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + 256 * i;
      pre[i] = cc * kScoreCols + e / D < T ? src[e] : 0.0;
    }
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + 256 * i;
      kbuf[buf][(e / D) * CS + e % D] = pre[i];
    }
  };
  if (c_lo >= c_hi) return;
  fetch(c_lo);
  put(0);
  __syncthreads();
  for (int cc = c_lo; cc < c_hi; ++cc) {
    const int buf = (cc - c_lo) & 1;
    if (cc + 1 < c_hi) fetch(cc + 1);  // in flight while this chunk is multiplied
    f64x4 acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = acc0;
    const double* kt = kbuf[buf];
#pragma unroll
    for (int s = 0; s < D / 4; ++s) {
      const double b0 = kt[l16 * CS + 4 * s + g];
      const double b1 = kt[(16 + l16) * CS + 4 * s + g];
      acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(af[s], b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(af[s], b1, acc1, 0, 0, 0);
    }
    // float64 16x16x4 accumulator: register i of lane group g holds row 4i + g
    const int c0 = cc * kScoreCols + l16, c1 = c0 + 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = rbase + 4 * i + g;
      if (rr < T) {
        if (c0 < T) out[(size_t)rr * T + c0] = acc0[i];
        if (c1 < T) out[(size_t)rr * T + c1] = acc1[i];
      }
    }
    if (cc + 1 < c_hi) put(buf ^ 1);  // that buffer was last read before the previous barrier
    __syncthreads();
  }
}

// -------------------------------------------------------------- top-k
// Order-preserving 64-bit key of a float64 (larger key <=> larger value;
// -0 is folded onto +0 so that equal values tie).
__device__ __forceinline__ uint64_t order_key(double x) {
  if (x == 0.0) x = 0.0;
  uint64_t u = (uint64_t)__double_as_longlong(x);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

constexpr int kMaxJ = 32;  // up to 64 * 32 = 2048 tiles per row (keys per lane: MJ <= kMaxJ)

// One wave per row: radix-select the k-th largest key (8 passes of 8 bits),
// keep every key above it and the lowest-index keys equal to it, add the
// diagonal if forced, and write the kept tiles in ascending order.
template <int MJ>  // keys per lane held in registers: T <= 64 * MJ
__global__ __launch_bounds__(256) void k_topk(int T, int rows, int topk, int force_diag, int direct,
                                              const double* __restrict__ scores, int32_t* __restrict__ out_cols,
                                              int32_t* __restrict__ out_cnt, int32_t* __restrict__ row_ptr) {
  __shared__ uint32_t hist[4][256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + w;
  const bool live = row < rows;
  const int a = live ? row % T : 0;
  const double* src = scores + (size_t)(live ? row : 0) * T;
  const int nj = (T + 63) / 64;

  uint64_t key[MJ];
#pragma unroll
  for (int j = 0; j < MJ; ++j) {
    int b = lane + 64 * j;
    key[j] = (j < nj && b < T && live) ? order_key(src[b]) : 0ull;
  }

  // Radix select of the k-th largest key.  After each pass, `prefix` holds the
  // bits fixed so far, `need` how many keys of that bucket are still needed.
  // When a bucket holds exactly the keys still needed, every key >= prefix is
  // kept and the search stops early (the usual case after two or three passes).
  // Each wave works on its own row and its own LDS histogram, so the waves of
  // a block never synchronise with each other.
  uint64_t prefix = 0, mask = 0;
  int need = topk;
  bool done = false;
  uint32_t* hw = hist[w];
  // First pass (sign and top exponent bits): the scores of a row fall into a
  // handful of these digits, so LDS atomics would serialise.  Walk the present
  // digits from the top instead, counting each with ballots, and stop at the
  // digit that holds the k-th key.
  {
    uint32_t pend = 0;
#pragma unroll
    for (int j = 0; j < MJ; ++j)
      if (j < nj && key[j] != 0ull) pend |= 1u << j;
    int cum = 0, digit = 0, dcnt = 0;
    for (;;) {
      int dl = -1;
#pragma unroll
      for (int j = 0; j < MJ; ++j)
        if ((pend >> j) & 1u) dl = max(dl, (int)(key[j] >> 56));
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) dl = max(dl, __shfl_xor(dl, off, 64));
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        if (j < nj) {
          const bool hit = ((pend >> j) & 1u) && (int)(key[j] >> 56) == dl;
          cnt += __popcll(__ballot(hit));
          if (hit) pend &= ~(1u << j);
        }
      }
      if (cum + cnt >= need || dl < 0) { digit = dl < 0 ? 0 : dl; dcnt = cnt; break; }
      cum += cnt;
    }
    need -= cum;
    prefix = (uint64_t)digit << 56;
    mask = 255ull << 56;
    done = dcnt == need;
  }
  for (int shift = 48; shift >= 0 && !done; shift -= 8) {
    for (int i = lane; i < 256; i += 64) hw[i] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < MJ; ++j)
      if (j < nj && (key[j] & mask) == prefix && key[j] != 0ull)
        atomicAdd(&hw[(key[j] >> shift) & 255u], 1u);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    __builtin_amdgcn_wave_barrier();
    // lane l owns digits 4l .. 4l+3; count from the top digit down
    const uint32_t h0 = hw[4 * lane], h1 = hw[4 * lane + 1], h2 = hw[4 * lane + 2], h3 = hw[4 * lane + 3];
    const uint32_t mine = h0 + h1 + h2 + h3;
    // inclusive suffix sum over lanes (lanes above hold larger digits)
    uint32_t suf = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_down(suf, off, 64);
      if (lane + off < 64) suf += o;
    }
    uint32_t cum = suf - mine;  // count in digits > 4l+3
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
    const int digit = __shfl(found, src_lane, 64);
    need = __shfl(rest, src_lane, 64);
    const int bcnt = __shfl(fcnt, src_lane, 64);
    prefix |= ((uint64_t)(digit < 0 ? 0 : digit)) << shift;
    mask |= 255ull << shift;
    done = bcnt == need;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
  }
  // keep key > kth, plus the `need` lowest-index keys equal to kth; an early
  // exit keeps every key >= prefix (kth = prefix - 1, no ties to break)
  const uint64_t kth = done ? prefix - 1 : prefix;
  if (done) need = 0;

  // selection flags: strictly above the threshold, then ties by lowest index
  uint32_t sel = 0;  // bit j: element j of this lane is kept
  int taken = 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int j = 0; j < MJ; ++j) {
    if (j < nj) {  // nj is wave-uniform; a guard instead of a break keeps key[] in registers
      const bool above = key[j] > kth;
      const bool eq = key[j] == kth && key[j] != 0ull;
      const uint64_t be = __ballot(eq);
      const int before = __popcll(be & lt_mask);
      if (above || (eq && taken + before < need)) sel |= 1u << j;
      taken += __popcll(be);
    }
  }
  if (force_diag && lane == (a & 63)) sel |= 1u << (a >> 6);

  // emit ascending
  int base_pos = 0;
  const size_t obase = direct ? (size_t)row * topk : (size_t)row * (topk + 1);
#pragma unroll
  for (int j = 0; j < MJ; ++j) {
    if (j < nj) {
      const bool s = (sel >> j) & 1u;
      const uint64_t bs = __ballot(s);
      if (s && live) out_cols[obase + base_pos + __popcll(bs & lt_mask)] = lane + 64 * j;
      base_pos += __popcll(bs);
    }
  }
  if (live && lane == 0) {
    if (direct) {
      row_ptr[row] = row * topk;
      if (row == rows - 1) row_ptr[rows] = rows * topk;
    } else {
      out_cnt[row] = base_pos;
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

hipError_t launch_scores(const Shape& s, const Scratch& w, hipStream_t st) {
  // Column parts (1..4): the split whose blocks fill the 512 block slots (two
  // blocks per CU) best over whole rounds, so that no last round runs mostly
  // empty (760 row blocks at 720P: 2 parts, 1520 blocks, 99% of 3 rounds).
  const long rowblocks = (long)((s.T + 63) / 64) * s.B * s.H;
  const int nch = (s.T + kScoreCols - 1) / kScoreCols;
  int parts = 1;
  double best = 0.0;
  for (int p = 1; p <= 4 && p <= nch; ++p) {
    const long blocks = rowblocks * p;
    const double fill = (double)blocks / (double)(((blocks + 511) / 512) * 512);
    if (fill > best + 1e-9) { best = fill; parts = p; }
  }
  dim3 g1((s.T + 63) / 64, s.B * s.H, parts);
  if (s.d == 64) k_scores<64><<<g1, 256, 0, st>>>(s.T, w.qmean, w.kmean, w.scores);
  else k_scores<128><<<g1, 256, 0, st>>>(s.T, w.qmean, w.kmean, w.scores);
  return hipGetLastError();
}

hipError_t launch_topk(const Shape& s, const Scratch& w, int32_t* row_ptr, int32_t* col_idx, hipStream_t st) {
  const int rows = s.B * s.H * s.T;
  hipError_t e;
  const int direct = s.force_diag ? 0 : 1;
  int32_t* cols = direct ? col_idx : w.sel_tmp;
  const int nj = (s.T + 63) / 64, grid = (rows + 3) / 4;
  if (nj <= 8) k_topk<8><<<grid, 256, 0, st>>>(s.T, rows, s.topk, s.force_diag, direct, w.scores, cols, w.sel_cnt, row_ptr);
  else if (nj <= 16) k_topk<16><<<grid, 256, 0, st>>>(s.T, rows, s.topk, s.force_diag, direct, w.scores, cols, w.sel_cnt, row_ptr);
  else if (nj <= 20) k_topk<20><<<grid, 256, 0, st>>>(s.T, rows, s.topk, s.force_diag, direct, w.scores, cols, w.sel_cnt, row_ptr);
  else k_topk<kMaxJ><<<grid, 256, 0, st>>>(s.T, rows, s.topk, s.force_diag, direct, w.scores, cols, w.sel_cnt, row_ptr);
  e = hipGetLastError();
  if (e != hipSuccess || direct) return e;
  k_scan<<<1, 1024, 0, st>>>(rows, w.sel_cnt, row_ptr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_compact<<<(rows + 255) / 256, 256, 0, st>>>(rows, s.topk + 1, w.sel_tmp, w.sel_cnt, row_ptr, col_idx);
  return hipGetLastError();
}

}  // namespace hsa
