// Internal interface between the C-ABI shim (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hsa {

enum class Dt : int { F32 = 0, BF16 = 1, FP8 = 2 };

// Layout of the bf16 hi and lo parts of the key tile means: the order of the
// selection's matrix-core B fragments.  Per (b, h): key block kb of 16 tiles,
// 32-wide d chunk c, then lane (tile mod 16) + 16 ((d mod 32) / 8), then 8
// consecutive d; one fragment load of a (kb, c) reads 1 KB contiguous.  The
// tiles are padded to whole key blocks (the padding holds zeros).
__host__ __device__ inline int kfrag_tiles(int T) { return 16 * ((T + 15) / 16); }
__host__ __device__ inline size_t kfrag_index(int t, int d, int D) {
  return ((size_t)((t >> 4) * (D / 32) + (d >> 5)) * 64 + ((d & 31) >> 3) * 16 + (t & 15)) * 8 + (d & 7);
}

// Position of element (row, col) of a row-major matrix with ncol columns in
// the fragment order the backward's linear kernels read their parameter
// operands in (one 1 KB or 2 KB run per fragment load): 16-row block, 32-wide
// column chunk (ceil(ncol / 32) per row block), lane (row mod 16) + 16 g,
// slot s, where slots 0-3 hold columns 32 c + 4 g + s and slots 4-7 columns
// 32 c + 16 + 4 g + (s - 4) (slots past ncol hold zeros).
__host__ __device__ inline size_t perm_frag_index(int row, int col, int ncol) {
  const int nch = (ncol + 31) / 32, c = col >> 5, wc = col & 31;
  const int g = (wc & 15) >> 2, s = (wc & 3) + (wc >= 16 ? 4 : 0);
  return ((size_t)((row >> 4) * nch + c) * 64 + g * 16 + (row & 15)) * 8 + s;
}
// The inverse: the (row, col) a fragment slot holds; col >= ncol marks a zero slot.
__host__ __device__ inline void perm_frag_source(size_t idx, int ncol, int* row, int* col) {
  const int nch = (ncol + 31) / 32, s = (int)(idx & 7), l = (int)((idx >> 3) & 63);
  const int fr = (int)(idx >> 9), c = fr % nch, g = l >> 4;
  *row = 16 * (fr / nch) + (l & 15);
  *col = 32 * c + (s < 4 ? 4 * g + s : 16 + 4 * g + (s - 4));
}

// Validated sizes as the kernels see them.
struct Shape {
  int B, H, N, N_pad, d, T;
  int gt, gh, gw;
  int topk, force_diag, kmax;
  int rank;
  float scale;      // softmax scale
  float rope_base;
  Dt dt;
  bool compl_keys;  // linear branch over the complement of each row's kept tiles
};

// Most tiles per (b, h) the complement variant handles (its per-block tile
// flags and index list live in LDS).
constexpr int kComplMaxT = 4096;

// RoPE table: for axis a (t, h, w) with D_a feature dims, the float2
// (cos, sin) of pos * base^(-2m/D_a) at tab[rope_off(a) + pos * D_a/2 + m].
inline int rope_dims(int rank, int axis) { return axis < 2 ? 3 * rank / 8 : rank / 4; }
inline int rope_entries(const Shape& s) {
  return s.gt * rope_dims(s.rank, 0) / 2 + s.gh * rope_dims(s.rank, 1) / 2 + s.gw * rope_dims(s.rank, 2) / 2;
}

// Number of tile chunks per (b, h) in the streaming pass.  The pass runs two
// 256-thread blocks per CU (512 on the 256 CUs); the chunk count makes the
// B*H*chunks blocks fill those slots in one round, so that no round runs
// half empty.  Chunks hold ceil(T / c) tiles each, and the count is then cut
// to the chunks that hold any tile: every chunk writes its partial state,
// which the finalize step sums over all of them.
inline int stream_chunks(const Shape& s) {
  constexpr int kSlots = 512;
  int c = kSlots / (s.B * s.H);
  if (c < 1) c = 1;
  if (c > s.T) c = s.T;
  const int per = (s.T + c - 1) / c;
  return (s.T + per - 1) / per;
}

// Device scratch of one call, carved out of the caller's workspace.
struct Scratch {
  double* qmean = nullptr;     // [BH][T][d] tile means of Q
  double* kmean = nullptr;     // [BH][T][d] tile means of K
  uint16_t* khi = nullptr;     // bf16 hi part of the key tile means, fragment order (kfrag_index)
  uint16_t* klo = nullptr;     // bf16 lo part, the same order
  int32_t* sel_tmp = nullptr;  // [BH*T][kmax] per-row selection (forced-diagonal path)
  int32_t* sel_cnt = nullptr;  // [BH*T]
  int32_t* row_ptr = nullptr;  // [BH*T + 1] internal CSR when the caller exports none
  int32_t* col_idx = nullptr;  // [BH*T*kmax]
  float* part_s = nullptr;     // [BH][chunks][r][d] partial states
  float* part_z = nullptr;     // [BH][chunks][r]
  void* sp_frag = nullptr;     // [BH] S' = S W_o as readout fragments (hi, lo)
  float* z = nullptr;          // [BH][r]
  void* uq_frag = nullptr;     // [H] U_q^T as readout fragments
  float2* rope = nullptr;      // RoPE table
  void* vt = nullptr;          // [BH][T][d][64] V tiles transposed, keys permuted (bf16 sparse path)
  void* tile_s = nullptr;      // complement variant: [BH][T] per-tile states as readout fragments
  float* tile_z = nullptr;     // [BH][T][r] per-tile feature sums
  float* s_full = nullptr;     // [BH] full state S (before W_o) as float readout fragments
  void* wo_frag = nullptr;     // [H] W_o^T as matrix-core A fragments
  // backward pass
  float* s_pfrag = nullptr;    // [BH][r*d] S (before W_o) in perm_frag_index order
  void* wob_frag = nullptr;    // [H][d*d] W_o as A fragments (rows 16-blocks, 32-wide column chunks)
  void* uqp_frag = nullptr;    // [H] U_q in perm_frag_index order
  void* ukp_frag = nullptr;    // [H] U_k in perm_frag_index order
  void* os = nullptr;          // [BH][N_pad][d] sparse-branch output, output type
  float* lse = nullptr;        // [BH][N_pad]
  float* dsum = nullptr;       // [BH][N_pad] dO . O_s
  float* part_ds = nullptr;    // [BH][chunks][r][d]
  float* part_dz = nullptr;    // [BH][chunks][r]
  float* ds_plain = nullptr;   // [BH][r][d]
  float* ds_frag = nullptr;    // [BH] dS^T as float readout fragments
  float* dz = nullptr;         // [BH][r]
  void* uk_frag = nullptr;     // [H] U_k^T as A fragments
  int32_t* csc_cnt = nullptr;  // [BH*T]
  int32_t* col_ptr = nullptr;  // [BH*T + 1]
  int32_t* row_idx = nullptr;  // [BH*T*T]
  uint32_t* csc_bits = nullptr;  // [BH*T][ceil(T/32)] transposed mask bits
  long csc_cap = 0;
};

// Workspace planning: byte offsets of each region for a given call.
struct Plan {
  size_t total = 0;
  size_t off_qmean = 0, off_kmean = 0, off_khi = 0, off_klo = 0, off_sel_tmp = 0, off_sel_cnt = 0;
  size_t off_row_ptr = 0, off_col_idx = 0, off_part_s = 0, off_part_z = 0, off_sp = 0;
  size_t off_z = 0, off_uq = 0, off_rope = 0, off_vt = 0;
  size_t off_tile_s = 0, off_tile_z = 0, off_s_full = 0, off_wo = 0;
  size_t off_s_pfrag = 0, off_wob = 0, off_uqp = 0, off_ukp = 0, off_os = 0, off_lse = 0, off_dsum = 0, off_part_ds = 0, off_part_dz = 0;
  size_t off_ds_plain = 0, off_ds_frag = 0, off_dz = 0, off_uk = 0, off_csc_cnt = 0, off_col_ptr = 0, off_row_idx = 0;
  size_t off_csc_bits = 0;
  bool select = false, csr_internal = false, linear = false, vt = false, compl_keys = false, backward = false;
};

Plan make_plan(const Shape& s, bool select, bool csr_internal, bool linear, bool vt, bool backward = false);

// Size of the static scratch behind hsa_hybrid_attn_noalloc, and its device
// address on the current device (taken on the first call there).
constexpr size_t kStaticScratchBytes = (size_t)256 << 20;  // HSA_ATTN_STATIC_SCRATCH_BYTES
hipError_t static_scratch(void** out);
Scratch bind_plan(const Plan& p, void* ws);

// Launchers: each enqueues its kernels on `st` and returns hipSuccess or the
// launch error.
constexpr int kReadCalibrateBlocks = 2048;  // blocks of 256 threads: one sink word per thread
hipError_t launch_read_calibrate(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st);
hipError_t launch_rope_table(const Shape& s, float2* tab, hipStream_t st);
hipError_t launch_stream_pass(const Shape& s, const void* q, const void* k, const void* v,
                              const float* qs, const float* ks, const float* vs,
                              const void* uk, bool pool, bool state, const Scratch& w,
                              double* kbar_out, hipStream_t st);
hipError_t launch_vtranspose(const Shape& s, const void* v, const Scratch& w, hipStream_t st);
hipError_t launch_finalize(const Shape& s, const void* uq, const void* wo, const Scratch& w, hipStream_t st);
// Selection: pooling of the query tiles, pooled scores, per-row top-k and the
// CSR (after a streaming pass that pooled the key tiles).
hipError_t launch_select(const Shape& s, const void* q, const float* qs, const Scratch& w, int32_t* row_ptr,
                         int32_t* col_idx, double* qbar_out, hipStream_t st);
hipError_t launch_attend(const Shape& s, const void* q, const void* k, const void* v,
                         const float* qs, const float* ks, const float* vs,
                         const int32_t* row_ptr, const int32_t* col_idx, bool sparse, bool linear,
                         const Scratch& w, void* o, float* lse, hipStream_t st, void* o_s = nullptr);
// Backward pass pieces (float32 gradients): part 1 = the linear branch (its dq,
// dk, dv written, D written), part 2 = the transposed mask and the sparse
// branch (dq, dk, dv added to).
hipError_t launch_backward(const Shape& s, const void* q, const void* k, const void* v, const void* dout,
                           const void* uq, const void* uk, const void* wo, const int32_t* row_ptr,
                           const int32_t* col_idx, const Scratch& w, float* dq, float* dk, float* dv, int part,
                           hipStream_t st);
// The complement variant's O_l W_o: added to o (which holds O_s) when `add`,
// else written to o.
hipError_t launch_compl(const Shape& s, const void* q, const float* qs, const int32_t* row_ptr,
                        const int32_t* col_idx, const Scratch& w, void* o, bool add, hipStream_t st);

}  // namespace hsa
