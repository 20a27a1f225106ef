// C-ABI shim: argument validation, workspace planning and launch order.
// Nothing is enqueued until every argument has been checked.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/hsa_attn.h"
#include "kernels.hpp"

#define HSA_API extern "C" __attribute__((visibility("default")))

namespace hsa {

static thread_local char g_err[512] = "";

static int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Plan make_plan(const Shape& s, bool select, bool csr_internal, bool linear, bool vt, bool backward) {
  Plan p;
  p.select = select; p.csr_internal = csr_internal; p.linear = linear || backward;
  p.backward = backward;
  linear = p.linear;
  p.compl_keys = linear && s.compl_keys;
  p.vt = vt && s.dt == Dt::FP8;  // the fp8 sparse kernel reads V pre-transposed
  const size_t bh = (size_t)s.B * s.H, rows = bh * s.T;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  if (select) {
    p.off_qmean = take(bh * s.d * s.T * sizeof(double));
    p.off_kmean = take(bh * s.d * s.T * sizeof(double));
    p.off_khi = take(bh * s.d * kfrag_tiles(s.T) * sizeof(uint16_t));
    p.off_klo = take(bh * s.d * kfrag_tiles(s.T) * sizeof(uint16_t));
    if (s.force_diag) {
      p.off_sel_tmp = take(rows * (s.topk + 1) * sizeof(int32_t));
      p.off_sel_cnt = take(rows * sizeof(int32_t));
    }
  }
  if (csr_internal) {
    p.off_row_ptr = take((rows + 1) * sizeof(int32_t));
    p.off_col_idx = take(rows * s.kmax * sizeof(int32_t));
  }
  if (linear) {
    const size_t elt = s.dt == Dt::F32 ? 4 : 2;
    const int nrc = (s.rank + 31) / 32, ndb = s.d / 16, nrb = s.rank / 16;
    const size_t nch = stream_chunks(s);
    p.off_part_s = take(bh * nch * s.rank * s.d * sizeof(float));
    p.off_part_z = take(bh * nch * s.rank * sizeof(float));
    p.off_sp = take(bh * (size_t)ndb * nrc * 512 * elt * (elt == 2 ? 2 : 1));
    p.off_z = take(bh * s.rank * sizeof(float));
    p.off_uq = take((size_t)s.H * nrb * (s.d / 32) * 512 * elt);
    p.off_rope = take((size_t)rope_entries(s) * sizeof(float2));
    if (p.compl_keys) {
      const size_t nfe = (size_t)ndb * nrc * 512;  // state elements as readout fragments
      p.off_tile_s = take(bh * s.T * nfe * elt);
      p.off_tile_z = take(bh * s.T * s.rank * sizeof(float));
      p.off_s_full = take(bh * nfe * sizeof(float));
      p.off_wo = take((size_t)s.H * s.d * s.d * elt);
    }
  }
  if (p.vt) p.off_vt = take(bh * (size_t)s.N_pad * s.d);  // one byte per code
  if (backward) {
    const size_t elt = s.dt == Dt::F32 ? 4 : 2;
    const int nrc = (s.rank + 31) / 32, ndb = s.d / 16, nrb = s.rank / 16;
    const size_t nfe = (size_t)ndb * nrc * 512, nch = stream_chunks(s), rd = (size_t)s.rank * s.d;
    if (!p.compl_keys) p.off_s_full = take(bh * nfe * sizeof(float));
    p.off_s_pfrag = take(bh * rd * sizeof(float));
    p.off_wob = take((size_t)s.H * s.d * s.d * elt);
    p.off_uqp = take((size_t)s.H * ndb * nrc * 512 * elt);
    p.off_ukp = take((size_t)s.H * ndb * nrc * 512 * elt);
    p.off_os = take(bh * (size_t)s.N_pad * s.d * elt);
    p.off_lse = take(bh * (size_t)s.N_pad * sizeof(float));
    p.off_dsum = take(bh * (size_t)s.N_pad * sizeof(float));
    p.off_part_ds = take(bh * nch * rd * sizeof(float));
    p.off_part_dz = take(bh * nch * s.rank * sizeof(float));
    p.off_ds_plain = take(bh * rd * sizeof(float));
    p.off_ds_frag = take(bh * nfe * sizeof(float));
    p.off_dz = take(bh * s.rank * sizeof(float));
    p.off_uk = take((size_t)s.H * nrb * (s.d / 32) * 512 * elt);
    p.off_csc_cnt = take(rows * sizeof(int32_t));
    p.off_col_ptr = take((rows + 1) * sizeof(int32_t));
    // the transposed mask holds as many entries as the mask: at most topk + force_diag per row
    p.off_row_idx = take(rows * (size_t)s.kmax * sizeof(int32_t));
    p.off_csc_bits = take(rows * (size_t)((s.T + 31) / 32) * sizeof(uint32_t));
  }
  p.total = off;
  return p;
}

Scratch bind_plan(const Plan& p, void* ws) {
  Scratch w;
  char* b = static_cast<char*>(ws);
  if (p.select) {
    w.qmean = reinterpret_cast<double*>(b + p.off_qmean);
    w.kmean = reinterpret_cast<double*>(b + p.off_kmean);
    w.khi = reinterpret_cast<uint16_t*>(b + p.off_khi);
    w.klo = reinterpret_cast<uint16_t*>(b + p.off_klo);
    w.sel_tmp = reinterpret_cast<int32_t*>(b + p.off_sel_tmp);
    w.sel_cnt = reinterpret_cast<int32_t*>(b + p.off_sel_cnt);
  }
  if (p.csr_internal) {
    w.row_ptr = reinterpret_cast<int32_t*>(b + p.off_row_ptr);
    w.col_idx = reinterpret_cast<int32_t*>(b + p.off_col_idx);
  }
  if (p.linear) {
    w.part_s = reinterpret_cast<float*>(b + p.off_part_s);
    w.part_z = reinterpret_cast<float*>(b + p.off_part_z);
    w.sp_frag = b + p.off_sp;
    w.z = reinterpret_cast<float*>(b + p.off_z);
    w.uq_frag = b + p.off_uq;
    w.rope = reinterpret_cast<float2*>(b + p.off_rope);
    if (p.compl_keys) {
      w.tile_s = b + p.off_tile_s;
      w.tile_z = reinterpret_cast<float*>(b + p.off_tile_z);
      w.s_full = reinterpret_cast<float*>(b + p.off_s_full);
      w.wo_frag = b + p.off_wo;
    }
  }
  if (p.vt) w.vt = b + p.off_vt;
  if (p.backward) {
    w.s_full = reinterpret_cast<float*>(b + p.off_s_full);
    w.s_pfrag = reinterpret_cast<float*>(b + p.off_s_pfrag);
    w.wob_frag = b + p.off_wob;
    w.uqp_frag = b + p.off_uqp;
    w.ukp_frag = b + p.off_ukp;
    w.os = b + p.off_os;
    w.lse = reinterpret_cast<float*>(b + p.off_lse);
    w.dsum = reinterpret_cast<float*>(b + p.off_dsum);
    w.part_ds = reinterpret_cast<float*>(b + p.off_part_ds);
    w.part_dz = reinterpret_cast<float*>(b + p.off_part_dz);
    w.ds_plain = reinterpret_cast<float*>(b + p.off_ds_plain);
    w.ds_frag = reinterpret_cast<float*>(b + p.off_ds_frag);
    w.dz = reinterpret_cast<float*>(b + p.off_dz);
    w.uk_frag = b + p.off_uk;
    w.csc_cnt = reinterpret_cast<int32_t*>(b + p.off_csc_cnt);
    w.col_ptr = reinterpret_cast<int32_t*>(b + p.off_col_ptr);
    w.row_idx = reinterpret_cast<int32_t*>(b + p.off_row_idx);
    w.csc_bits = reinterpret_cast<uint32_t*>(b + p.off_csc_bits);
  }
  return w;
}

// Checks a descriptor; `need_rank` when the linear branch runs, `need_select`
// when tiles are selected.
static int check_desc(const hsa_attn_desc* d, Shape& s, bool need_rank, bool need_select) {
  if (!d) return fail(HSA_ATTN_ERR_NULL, "desc is NULL");
  if (d->B < 1 || d->H < 1) return fail(HSA_ATTN_ERR_SHAPE, "B=%d H=%d must be >= 1", d->B, d->H);
  if (d->tile != 64) return fail(HSA_ATTN_ERR_SHAPE, "tile=%d: only 64 is supported", d->tile);
  if (d->d != 64 && d->d != 128) return fail(HSA_ATTN_ERR_SHAPE, "d=%d: only 64 and 128 are supported", d->d);
  if (d->N < 1) return fail(HSA_ATTN_ERR_SHAPE, "N=%d must be >= 1", d->N);
  if (d->N_pad % 64 != 0 || d->N_pad < d->N || d->N_pad - d->N >= 64)
    return fail(HSA_ATTN_ERR_SHAPE, "N_pad=%d must be the multiple of 64 in [N, N+63] (N=%d)", d->N_pad, d->N);
  if (d->grid_t < 1 || d->grid_h < 1 || d->grid_w < 1 || d->grid_h >= 1024 || d->grid_w >= 1024 || d->grid_t >= 2048)
    return fail(HSA_ATTN_ERR_SHAPE, "grid %dx%dx%d out of range (t < 2048, h and w < 1024)", d->grid_t, d->grid_h, d->grid_w);
  if ((long long)d->grid_t * d->grid_h * d->grid_w != d->N)
    return fail(HSA_ATTN_ERR_SHAPE, "grid %dx%dx%d does not hold N=%d tokens", d->grid_t, d->grid_h, d->grid_w, d->N);
  // The kernels address one (b, h) slice with 32-bit byte offsets and buffer
  // sizes; the widest tensor a call touches per slice is float32 (backward
  // gradients, float32 inputs), so N_pad * d * 4 bytes must stay below 2^31.
  if ((long long)d->N_pad * d->d * 4 >= (1ll << 31))
    return fail(HSA_ATTN_ERR_SHAPE, "N_pad=%d x d=%d: one (b, h) slice of float32 must stay below 2^31 bytes",
                d->N_pad, d->d);
  const int T = d->N_pad / 64;
  if (need_select && T > 2048) return fail(HSA_ATTN_ERR_SHAPE, "T=%d tiles per row: selection supports at most 2048", T);
  if (need_select && (d->topk < 1 || d->topk > T)) return fail(HSA_ATTN_ERR_SHAPE, "topk=%d must be in [1, T=%d]", d->topk, T);
  if (d->force_diag != 0 && d->force_diag != 1) return fail(HSA_ATTN_ERR_SHAPE, "force_diag=%d must be 0 or 1", d->force_diag);
  if (need_rank && d->rank != 16 && d->rank != 32 && d->rank != 64)
    return fail(HSA_ATTN_ERR_SHAPE, "rank=%d: supported ranks are 16, 32, 64", d->rank);
  if (!(isfinite(d->softmax_scale) && d->softmax_scale > 0.f))
    return fail(HSA_ATTN_ERR_SHAPE, "softmax_scale must be finite and > 0");
  if (need_rank && !(d->rope_base > 0.f && isfinite(d->rope_base))) return fail(HSA_ATTN_ERR_SHAPE, "rope_base must be > 0");
  const bool ok_dt = (d->in_dtype == HSA_ATTN_F32 && d->out_dtype == HSA_ATTN_F32) ||
                     (d->in_dtype == HSA_ATTN_BF16 && d->out_dtype == HSA_ATTN_BF16) ||
                     (d->in_dtype == HSA_ATTN_FP8_E4M3 && d->out_dtype == HSA_ATTN_BF16);
  if (!ok_dt) return fail(HSA_ATTN_ERR_DTYPE, "dtype pair (%d, %d) unsupported: use (F32,F32), (BF16,BF16) or (FP8_E4M3,BF16)",
                          d->in_dtype, d->out_dtype);
  if (d->linear_keys != HSA_ATTN_LINEAR_ALL_KEYS && d->linear_keys != HSA_ATTN_LINEAR_COMPLEMENT)
    return fail(HSA_ATTN_ERR_SHAPE, "linear_keys=%d must be 0 (all keys) or 1 (complement)", d->linear_keys);
  if (need_rank && d->linear_keys == HSA_ATTN_LINEAR_COMPLEMENT && T > kComplMaxT)
    return fail(HSA_ATTN_ERR_SHAPE, "T=%d tiles: the complement variant supports at most %d", T, kComplMaxT);
  const long long rows = (long long)d->B * d->H * T;
  if (rows * (d->topk + 1) >= (1ll << 31)) return fail(HSA_ATTN_ERR_SHAPE, "B*H*T*(topk+1) exceeds int32 CSR range");
  s.B = d->B; s.H = d->H; s.N = d->N; s.N_pad = d->N_pad; s.d = d->d; s.T = T;
  s.gt = d->grid_t; s.gh = d->grid_h; s.gw = d->grid_w;
  s.topk = d->topk; s.force_diag = d->force_diag; s.kmax = d->topk + d->force_diag;
  s.rank = d->rank; s.scale = d->softmax_scale; s.rope_base = d->rope_base;
  s.dt = static_cast<Dt>(d->in_dtype);
  s.compl_keys = d->linear_keys == HSA_ATTN_LINEAR_COMPLEMENT;
  return HSA_ATTN_OK;
}

static int check_scales(const Shape& s, const float* a, const float* b, const float* c, int nneeded) {
  const float* p[3] = {a, b, c};
  for (int i = 0; i < 3; ++i) {
    if (s.dt == Dt::FP8 && i < nneeded && !p[i]) return fail(HSA_ATTN_ERR_DTYPE, "FP8 inputs need their scale arrays");
    if (s.dt != Dt::FP8 && p[i]) return fail(HSA_ATTN_ERR_DTYPE, "scale arrays are only for FP8 inputs");
  }
  return HSA_ATTN_OK;
}

static int check_ws(const Plan& p, void* ws, size_t bytes) {
  if (p.total == 0) return HSA_ATTN_OK;
  if (!ws) return fail(HSA_ATTN_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", p.total);
  if (bytes < p.total) return fail(HSA_ATTN_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu needed", bytes, p.total);
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(HSA_ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return HSA_ATTN_OK;
}

static int hip_fail(hipError_t e, const char* what) {
  return fail(HSA_ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ----------------------------------------------------------------- timing
// Optional per-kernel timing with HIP events recorded on the launch stream.
struct Timing {
  std::mutex mu;
  int max = 0;
  int count[HSA_ATTN_KERNEL_KINDS] = {};
  std::vector<hipEvent_t> ev[HSA_ATTN_KERNEL_KINDS];  // start/stop pairs
  hipEvent_t last = nullptr;
};
static Timing g_timing;

template <class F>
static hipError_t timed(int kind, hipStream_t st, F&& launch) {
  int idx = -1;
  {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (g_timing.max > 0 && g_timing.count[kind] < g_timing.max) {
      idx = g_timing.count[kind]++;
      hipEventRecord(g_timing.ev[kind][2 * idx], st);
    }
  }
  hipError_t e = launch();
  if (idx >= 0) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    hipEventRecord(g_timing.ev[kind][2 * idx + 1], st);
    g_timing.last = g_timing.ev[kind][2 * idx + 1];
  }
  return e;
}

}  // namespace hsa

using namespace hsa;

HSA_API const char* hsa_attn_last_error(void) { return g_err; }

HSA_API const char* hsa_attn_version(void) { return "hsa_attn 0.1 gfx950"; }

HSA_API int hsa_attn_timing_enable(int max_launches) {
  if (max_launches < 0) return fail(HSA_ATTN_ERR_SHAPE, "max_launches must be >= 0");
  std::lock_guard<std::mutex> lk(g_timing.mu);
  for (int k = 0; k < HSA_ATTN_KERNEL_KINDS; ++k) {
    for (hipEvent_t e : g_timing.ev[k]) hipEventDestroy(e);
    g_timing.ev[k].clear();
    g_timing.count[k] = 0;
  }
  g_timing.last = nullptr;
  g_timing.max = 0;
  for (int k = 0; k < HSA_ATTN_KERNEL_KINDS; ++k) {
    g_timing.ev[k].resize(2 * (size_t)max_launches);
    for (auto& e : g_timing.ev[k]) {
      hipError_t rc = hipEventCreate(&e);
      if (rc != hipSuccess) return hip_fail(rc, "hipEventCreate");
    }
  }
  g_timing.max = max_launches;
  return HSA_ATTN_OK;
}

HSA_API int hsa_attn_read_calibrate(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words,
                                    void* stream) {
  if (!buf || !sink) return fail(HSA_ATTN_ERR_NULL, "read_calibrate: buf and sink are required");
  if (bytes == 0 || bytes % 16 != 0)
    return fail(HSA_ATTN_ERR_SHAPE, "read_calibrate: bytes=%zu must be a positive multiple of 16", bytes);
  if (sink_words < (size_t)HSA_ATTN_READ_SINK_WORDS)
    return fail(HSA_ATTN_ERR_SHAPE, "read_calibrate: sink holds %zu words, %d are needed", sink_words,
                HSA_ATTN_READ_SINK_WORDS);
  hipError_t e = hsa::launch_read_calibrate(buf, bytes, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "read calibration");
  return HSA_ATTN_OK;
}

HSA_API int hsa_attn_timing_read(double* ms_out, int32_t* launches_out) {
  if (!ms_out || !launches_out) return fail(HSA_ATTN_ERR_NULL, "ms_out and launches_out are required");
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (g_timing.last) {
    hipError_t rc = hipEventSynchronize(g_timing.last);
    if (rc != hipSuccess) return hip_fail(rc, "hipEventSynchronize");
  }
  for (int k = 0; k < HSA_ATTN_KERNEL_KINDS; ++k) {
    double sum = 0.0;
    for (int i = 0; i < g_timing.count[k]; ++i) {
      float ms = 0.f;
      hipError_t rc = hipEventElapsedTime(&ms, g_timing.ev[k][2 * i], g_timing.ev[k][2 * i + 1]);
      if (rc != hipSuccess) return hip_fail(rc, "hipEventElapsedTime");
      sum += ms;
    }
    ms_out[k] = sum;
    launches_out[k] = g_timing.count[k];
  }
  return HSA_ATTN_OK;
}

// The backward pass covers float32 and bf16 inputs and the all-keys linear branch.
static int check_backward(const Shape& s) {
  if (s.dt == Dt::FP8) return fail(HSA_ATTN_ERR_DTYPE, "the backward pass takes float32 or bf16 inputs");
  if (s.compl_keys) return fail(HSA_ATTN_ERR_SHAPE, "the backward pass covers the all-keys linear branch only");
  if (s.topk < 1 || s.topk > s.T) return fail(HSA_ATTN_ERR_SHAPE, "topk=%d must be in [1, T=%d]", s.topk, s.T);
  return HSA_ATTN_OK;
}

HSA_API int hsa_attn_workspace_size(const hsa_attn_desc* desc, int call, size_t* bytes) {
  if (!bytes) return fail(HSA_ATTN_ERR_NULL, "bytes is NULL");
  Shape s;
  const bool lin = call == HSA_ATTN_CALL_LINEAR || call == HSA_ATTN_CALL_HYBRID ||
                   call == HSA_ATTN_CALL_LINEAR_COMPLEMENT || call == HSA_ATTN_CALL_BACKWARD;
  const bool sel = call == HSA_ATTN_CALL_BLOCK_SELECT || call == HSA_ATTN_CALL_HYBRID;
  if (call < 0 || call > 5) return fail(HSA_ATTN_ERR_SHAPE, "unknown call %d", call);
  int rc = check_desc(desc, s, lin, sel);
  if (rc) return rc;
  if (call == HSA_ATTN_CALL_LINEAR && s.compl_keys)
    return fail(HSA_ATTN_ERR_SHAPE, "the complement variant needs a mask: use hsa_linear_attn_complement");
  if (call == HSA_ATTN_CALL_LINEAR_COMPLEMENT) {
    if (s.T > kComplMaxT) return fail(HSA_ATTN_ERR_SHAPE, "T=%d tiles: the complement variant supports at most %d", s.T, kComplMaxT);
    s.compl_keys = true;
  }
  if (call == HSA_ATTN_CALL_BACKWARD) {
    if ((rc = check_backward(s))) return rc;
    *bytes = make_plan(s, false, false, true, false, true).total;
    return HSA_ATTN_OK;
  }
  // the hybrid figure covers its largest variant (selection + internal CSR)
  const bool sparse = call == HSA_ATTN_CALL_SPARSE || call == HSA_ATTN_CALL_HYBRID;
  *bytes = make_plan(s, sel, call == HSA_ATTN_CALL_HYBRID, lin, sparse).total;
  return HSA_ATTN_OK;
}

HSA_API int hsa_block_select(const hsa_attn_desc* desc, const void* q, const void* k,
                             const float* q_scale, const float* k_scale,
                             int32_t* row_ptr, int32_t* col_idx, double* qbar_out, double* kbar_out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  int rc = check_desc(desc, s, false, true);
  if (rc) return rc;
  if (!q || !k || !row_ptr || !col_idx) return fail(HSA_ATTN_ERR_NULL, "q, k, row_ptr and col_idx are required");
  if ((rc = check_scales(s, q_scale, k_scale, nullptr, 2))) return rc;
  Plan p = make_plan(s, true, false, false, false);
  if ((rc = check_ws(p, workspace, workspace_bytes))) return rc;
  Scratch w = bind_plan(p, workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = timed(HSA_ATTN_KERNEL_STREAM, st, [&] {
    return launch_stream_pass(s, nullptr, k, nullptr, nullptr, k_scale, nullptr, nullptr, true, false, w, kbar_out,
                              st);
  });
  if (e != hipSuccess) return hip_fail(e, "key tile pooling");
  e = timed(HSA_ATTN_KERNEL_SELECT, st, [&] {
    return launch_select(s, q, q_scale, w, row_ptr, col_idx, qbar_out, st);
  });
  if (e != hipSuccess) return hip_fail(e, "tile selection");
  return HSA_ATTN_OK;
}

HSA_API int hsa_sparse_attn(const hsa_attn_desc* desc, const void* q, const void* k, const void* v,
                            const float* q_scale, const float* k_scale, const float* v_scale,
                            const int32_t* row_ptr, const int32_t* col_idx, void* o_sparse, float* lse_out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  int rc = check_desc(desc, s, false, false);
  if (rc) return rc;
  if (!q || !k || !v || !row_ptr || !col_idx || !o_sparse)
    return fail(HSA_ATTN_ERR_NULL, "q, k, v, row_ptr, col_idx and o_sparse are required");
  if ((rc = check_scales(s, q_scale, k_scale, v_scale, 3))) return rc;
  if (s.dt == Dt::FP8 && s.d != 128) return fail(HSA_ATTN_ERR_SHAPE, "FP8 attention needs head dim 128 (d=%d)", s.d);
  Plan p = make_plan(s, false, false, false, true);
  if ((rc = check_ws(p, workspace, workspace_bytes))) return rc;
  Scratch w = bind_plan(p, workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (p.vt) {
    e = timed(HSA_ATTN_KERNEL_STREAM, st, [&] { return launch_vtranspose(s, v, w, st); });
    if (e != hipSuccess) return hip_fail(e, "V transpose");
  }
  e = timed(HSA_ATTN_KERNEL_ATTEND, st, [&] {
    return launch_attend(s, q, k, v, q_scale, k_scale, v_scale, row_ptr, col_idx, true, false, w, o_sparse,
                         lse_out, st);
  });
  if (e != hipSuccess) return hip_fail(e, "sparse attention");
  return HSA_ATTN_OK;
}

static int run_linear_state(const Shape& s, const void* q, const void* k, const void* v,
                            const float* qs, const float* ks, const float* vs,
                            const void* uq, const void* uk, const void* wo, bool pool, const Scratch& w,
                            hipStream_t st) {
  hipError_t e = timed(HSA_ATTN_KERNEL_ROPE, st, [&] { return launch_rope_table(s, w.rope, st); });
  if (e != hipSuccess) return hip_fail(e, "rope table");
  e = timed(HSA_ATTN_KERNEL_STREAM, st, [&] {
    return launch_stream_pass(s, q, k, v, qs, ks, vs, uk, pool, true, w, nullptr, st);
  });
  if (e != hipSuccess) return hip_fail(e, "streaming pass");
  e = timed(HSA_ATTN_KERNEL_FINALIZE, st, [&] { return launch_finalize(s, uq, wo, w, st); });
  if (e != hipSuccess) return hip_fail(e, "state finalize");
  return HSA_ATTN_OK;
}

HSA_API int hsa_linear_attn(const hsa_attn_desc* desc, const void* q, const void* k, const void* v,
                            const float* q_scale, const float* k_scale, const float* v_scale,
                            const void* U_q, const void* U_k, const void* W_o, void* o_lin,
                            void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  int rc = check_desc(desc, s, true, false);
  if (rc) return rc;
  if (s.compl_keys)
    return fail(HSA_ATTN_ERR_SHAPE, "the complement variant needs a mask: use hsa_linear_attn_complement");
  if (!q || !k || !v || !U_q || !U_k || !W_o || !o_lin)
    return fail(HSA_ATTN_ERR_NULL, "q, k, v, U_q, U_k, W_o and o_lin are required");
  if ((rc = check_scales(s, q_scale, k_scale, v_scale, 3))) return rc;
  if (s.dt == Dt::FP8 && s.d != 128) return fail(HSA_ATTN_ERR_SHAPE, "FP8 attention needs head dim 128 (d=%d)", s.d);
  Plan p = make_plan(s, false, false, true, false);
  if ((rc = check_ws(p, workspace, workspace_bytes))) return rc;
  Scratch w = bind_plan(p, workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((rc = run_linear_state(s, q, k, v, q_scale, k_scale, v_scale, U_q, U_k, W_o, false, w, st))) return rc;
  hipError_t e = timed(HSA_ATTN_KERNEL_ATTEND, st, [&] {
    return launch_attend(s, q, k, v, q_scale, k_scale, v_scale, nullptr, nullptr, false, true, w, o_lin, nullptr, st);
  });
  if (e != hipSuccess) return hip_fail(e, "linear readout");
  return HSA_ATTN_OK;
}

HSA_API int hsa_linear_attn_complement(const hsa_attn_desc* desc, const void* q, const void* k, const void* v,
                                       const float* q_scale, const float* k_scale, const float* v_scale,
                                       const void* U_q, const void* U_k, const void* W_o,
                                       const int32_t* row_ptr, const int32_t* col_idx, void* o_lin,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  int rc = check_desc(desc, s, true, false);
  if (rc) return rc;
  if (s.T > kComplMaxT) return fail(HSA_ATTN_ERR_SHAPE, "T=%d tiles: the complement variant supports at most %d", s.T, kComplMaxT);
  s.compl_keys = true;  // this call always sums over the complement
  if (!q || !k || !v || !U_q || !U_k || !W_o || !o_lin)
    return fail(HSA_ATTN_ERR_NULL, "q, k, v, U_q, U_k, W_o and o_lin are required");
  if (!row_ptr || !col_idx) return fail(HSA_ATTN_ERR_CSR, "row_ptr and col_idx are required");
  if ((rc = check_scales(s, q_scale, k_scale, v_scale, 3))) return rc;
  if (s.dt == Dt::FP8 && s.d != 128) return fail(HSA_ATTN_ERR_SHAPE, "FP8 attention needs head dim 128 (d=%d)", s.d);
  Plan p = make_plan(s, false, false, true, false);
  if ((rc = check_ws(p, workspace, workspace_bytes))) return rc;
  Scratch w = bind_plan(p, workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((rc = run_linear_state(s, q, k, v, q_scale, k_scale, v_scale, U_q, U_k, W_o, false, w, st))) return rc;
  hipError_t e = timed(HSA_ATTN_KERNEL_COMPL, st, [&] {
    return launch_compl(s, q, q_scale, row_ptr, col_idx, w, o_lin, false, st);
  });
  if (e != hipSuccess) return hip_fail(e, "complement linear branch");
  return HSA_ATTN_OK;
}

// The hybrid call with its workspace either given by the caller or, for the
// allocation-free entry point (noalloc), the library's static scratch.
static int hybrid_impl(const hsa_attn_desc* desc, const void* q, const void* k, const void* v,
                       const float* q_scale, const float* k_scale, const float* v_scale,
                       const void* U_q, const void* U_k, const void* W_o,
                       const int32_t* row_ptr_in, const int32_t* col_idx_in,
                       int32_t* row_ptr_out, int32_t* col_idx_out,
                       void* o, void* workspace, size_t workspace_bytes, void* stream, bool noalloc,
                       void* o_s = nullptr, float* lse = nullptr) {
  Shape s;
  const bool given = row_ptr_in || col_idx_in;
  if (given && !(row_ptr_in && col_idx_in)) return fail(HSA_ATTN_ERR_CSR, "row_ptr_in and col_idx_in go together");
  if ((row_ptr_out || col_idx_out) && !(row_ptr_out && col_idx_out))
    return fail(HSA_ATTN_ERR_CSR, "row_ptr_out and col_idx_out go together");
  if (given && row_ptr_out) return fail(HSA_ATTN_ERR_CSR, "a given mask cannot also be exported");
  int rc = check_desc(desc, s, true, !given);
  if (rc) return rc;
  if (!q || !k || !v || !U_q || !U_k || !W_o || !o)
    return fail(HSA_ATTN_ERR_NULL, "q, k, v, U_q, U_k, W_o and o are required");
  if ((rc = check_scales(s, q_scale, k_scale, v_scale, 3))) return rc;
  if (s.dt == Dt::FP8 && s.d != 128) return fail(HSA_ATTN_ERR_SHAPE, "FP8 attention needs head dim 128 (d=%d)", s.d);
  const bool internal = !given && !row_ptr_out;
  Plan p = make_plan(s, !given, internal, true, true);
  if (noalloc) {
    if (p.total > kStaticScratchBytes)
      return fail(HSA_ATTN_ERR_WORKSPACE, "this call needs %zu bytes of scratch; the static scratch holds %zu",
                  p.total, kStaticScratchBytes);
    hipError_t e = static_scratch(&workspace);
    if (e != hipSuccess) return hip_fail(e, "static scratch address");
    workspace_bytes = kStaticScratchBytes;
  }
  if ((rc = check_ws(p, workspace, workspace_bytes))) return rc;
  Scratch w = bind_plan(p, workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((rc = run_linear_state(s, q, k, v, q_scale, k_scale, v_scale, U_q, U_k, W_o, !given, w, st))) return rc;
  const int32_t* rp = row_ptr_in;
  const int32_t* ci = col_idx_in;
  if (!given) {
    int32_t* rpo = internal ? w.row_ptr : row_ptr_out;
    int32_t* cio = internal ? w.col_idx : col_idx_out;
    hipError_t e = timed(HSA_ATTN_KERNEL_SELECT, st, [&] {
      return launch_select(s, q, q_scale, w, rpo, cio, nullptr, st);
    });
    if (e != hipSuccess) return hip_fail(e, "tile selection");
    rp = rpo;
    ci = cio;
  }
  // all keys: the query-tile kernel also reads the linear branch out; the
  // complement variant adds its own readout to the sparse output afterwards
  hipError_t e = timed(HSA_ATTN_KERNEL_ATTEND, st, [&] {
    return launch_attend(s, q, k, v, q_scale, k_scale, v_scale, rp, ci, true, !s.compl_keys, w, o, lse, st, o_s);
  });
  if (e != hipSuccess) return hip_fail(e, "hybrid attention");
  if (s.compl_keys) {
    e = timed(HSA_ATTN_KERNEL_COMPL, st, [&] { return launch_compl(s, q, q_scale, rp, ci, w, o, true, st); });
    if (e != hipSuccess) return hip_fail(e, "complement linear branch");
  }
  return HSA_ATTN_OK;
}

HSA_API int hsa_hybrid_attn(const hsa_attn_desc* desc, const void* q, const void* k, const void* v,
                            const float* q_scale, const float* k_scale, const float* v_scale,
                            const void* U_q, const void* U_k, const void* W_o,
                            const int32_t* row_ptr_in, const int32_t* col_idx_in,
                            int32_t* row_ptr_out, int32_t* col_idx_out,
                            void* o, void* workspace, size_t workspace_bytes, void* stream) {
  return hybrid_impl(desc, q, k, v, q_scale, k_scale, v_scale, U_q, U_k, W_o, row_ptr_in, col_idx_in, row_ptr_out,
                     col_idx_out, o, workspace, workspace_bytes, stream, false);
}

static_assert(kStaticScratchBytes == HSA_ATTN_STATIC_SCRATCH_BYTES, "static scratch size");

HSA_API int hsa_hybrid_attn_noalloc(const hsa_attn_desc* desc, const void* q, const void* k, const void* v,
                                    const float* q_scale, const float* k_scale, const float* v_scale,
                                    const void* U_q, const void* U_k, const void* W_o,
                                    const int32_t* row_ptr_in, const int32_t* col_idx_in,
                                    int32_t* row_ptr_out, int32_t* col_idx_out, void* o, void* stream) {
  return hybrid_impl(desc, q, k, v, q_scale, k_scale, v_scale, U_q, U_k, W_o, row_ptr_in, col_idx_in, row_ptr_out,
                     col_idx_out, o, nullptr, 0, stream, true);
}

HSA_API int hsa_hybrid_attn_train(const hsa_attn_desc* desc, const void* q, const void* k, const void* v,
                                  const void* U_q, const void* U_k, const void* W_o,
                                  const int32_t* row_ptr_in, const int32_t* col_idx_in,
                                  int32_t* row_ptr_out, int32_t* col_idx_out, void* o, void* o_s, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  int rc = check_desc(desc, s, true, false);
  if (rc) return rc;
  if ((rc = check_backward(s))) return rc;  // the calls whose gradients the backward gives
  if (!o_s || !lse) return fail(HSA_ATTN_ERR_NULL, "o_s and lse are required");
  return hybrid_impl(desc, q, k, v, nullptr, nullptr, nullptr, U_q, U_k, W_o, row_ptr_in, col_idx_in, row_ptr_out,
                     col_idx_out, o, workspace, workspace_bytes, stream, false, o_s, lse);
}

// ---------------------------------------------------------------- W8A8 projections
namespace hsa {
hipError_t launch_quant_rows(const void* x, long M, int C, void* codes, float* scales, hipStream_t st);
hipError_t launch_proj_fp8(const void* x, const float* sx, const void* wq, const float* sw, long M, int C, int H,
                           int n_pad, void* const* out, float* const* osc, hipStream_t st);
}  // namespace hsa

HSA_API int hsa_quantize_rows_fp8(const void* x, int64_t M, int64_t C, void* codes_out, float* scales_out,
                                  void* stream) {
  if (M < 0 || C <= 0 || C % 8 != 0 || C > (1 << 30))
    return fail(HSA_ATTN_ERR_SHAPE, "quantize_rows: C must be a positive multiple of 8 and M >= 0 (M=%lld C=%lld)",
                (long long)M, (long long)C);
  if (M > 0 && (!x || !codes_out || !scales_out))
    return fail(HSA_ATTN_ERR_NULL, "quantize_rows: x, codes_out and scales_out are required");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = timed(HSA_ATTN_KERNEL_QUANT, st, [&] {
    return launch_quant_rows(x, (long)M, (int)C, codes_out, scales_out, st);
  });
  if (e != hipSuccess) return hip_fail(e, "row quantisation");
  return HSA_ATTN_OK;
}

HSA_API int hsa_qkv_proj_fp8(const void* x_codes, const float* x_scales, const void* w_codes, const float* w_scales,
                             int32_t B, int32_t N_pad, int32_t C, int32_t H, int32_t d,
                             void* q, void* k, void* v, float* q_scales, float* k_scales, float* v_scales,
                             void* stream) {
  if (d != 128) return fail(HSA_ATTN_ERR_SHAPE, "qkv_proj: head dim must be 128 (d=%d)", d);
  if (B < 1 || H < 1 || N_pad < 64 || N_pad % 64 != 0)
    return fail(HSA_ATTN_ERR_SHAPE, "qkv_proj: need B, H >= 1 and N_pad a positive multiple of 64 (B=%d H=%d N_pad=%d)",
                B, H, N_pad);
  if (C < 128 || C % 128 != 0 || (long long)256 * C >= (1LL << 31))
    return fail(HSA_ATTN_ERR_SHAPE, "qkv_proj: C must be a multiple of 128 with 256*C < 2^31 (C=%d)", C);
  if (!x_codes || !x_scales || !w_codes || !w_scales || !q || !k || !v || !q_scales || !k_scales || !v_scales)
    return fail(HSA_ATTN_ERR_NULL, "qkv_proj: every pointer is required");
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* out[3] = {q, k, v};
  float* osc[3] = {q_scales, k_scales, v_scales};
  hipError_t e = timed(HSA_ATTN_KERNEL_PROJ, st, [&] {
    return launch_proj_fp8(x_codes, x_scales, w_codes, w_scales, (long)B * N_pad, C, H, N_pad, out, osc, st);
  });
  if (e != hipSuccess) return hip_fail(e, "qkv projection");
  return HSA_ATTN_OK;
}

// ---------------------------------------------------------------- backward
static int backward_impl(const hsa_attn_desc* desc, const void* q, const void* k, const void* v,
                         const void* U_q, const void* U_k, const void* W_o,
                         const int32_t* row_ptr, const int32_t* col_idx, const void* o_s, const float* lse,
                         const void* d_o, float* d_q, float* d_k, float* d_v,
                         void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  int rc = check_desc(desc, s, true, false);
  if (rc) return rc;
  if ((rc = check_backward(s))) return rc;
  if (!q || !k || !v || !U_q || !U_k || !W_o || !d_o || !d_q || !d_k || !d_v)
    return fail(HSA_ATTN_ERR_NULL, "q, k, v, U_q, U_k, W_o, d_o, d_q, d_k and d_v are required");
  if (!row_ptr || !col_idx) return fail(HSA_ATTN_ERR_CSR, "row_ptr and col_idx are required");
  Plan p = make_plan(s, false, false, true, false, true);
  if ((rc = check_ws(p, workspace, workspace_bytes))) return rc;
  Scratch w = bind_plan(p, workspace);
  w.csc_cap = (long)s.B * s.H * s.T * s.kmax;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the forward state (S, z), recomputed; the sparse branch's output and
  // log-sum-exp as the training forward saved them, or recomputed
  if ((rc = run_linear_state(s, q, k, v, nullptr, nullptr, nullptr, U_q, U_k, W_o, false, w, st))) return rc;
  hipError_t e;
  if (o_s) {
    w.os = const_cast<void*>(o_s);
    w.lse = const_cast<float*>(lse);
  } else {
    e = timed(HSA_ATTN_KERNEL_ATTEND, st, [&] {
      return launch_attend(s, q, k, v, nullptr, nullptr, nullptr, row_ptr, col_idx, true, false, w, w.os, w.lse, st);
    });
    if (e != hipSuccess) return hip_fail(e, "sparse recompute");
  }
  e = timed(HSA_ATTN_KERNEL_BWD_LINEAR, st, [&] {
    return launch_backward(s, q, k, v, d_o, U_q, U_k, W_o, row_ptr, col_idx, w, d_q, d_k, d_v, 1, st);
  });
  if (e != hipSuccess) return hip_fail(e, "linear backward");
  e = timed(HSA_ATTN_KERNEL_BWD_SPARSE, st, [&] {
    return launch_backward(s, q, k, v, d_o, U_q, U_k, W_o, row_ptr, col_idx, w, d_q, d_k, d_v, 2, st);
  });
  if (e != hipSuccess) return hip_fail(e, "sparse backward");
  return HSA_ATTN_OK;
}

HSA_API int hsa_hybrid_attn_backward(const hsa_attn_desc* desc, const void* q, const void* k, const void* v,
                                     const void* U_q, const void* U_k, const void* W_o,
                                     const int32_t* row_ptr, const int32_t* col_idx, const void* d_o,
                                     float* d_q, float* d_k, float* d_v,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(desc, q, k, v, U_q, U_k, W_o, row_ptr, col_idx, nullptr, nullptr, d_o, d_q, d_k, d_v,
                       workspace, workspace_bytes, stream);
}

HSA_API int hsa_hybrid_attn_backward_saved(const hsa_attn_desc* desc, const void* q, const void* k, const void* v,
                                           const void* U_q, const void* U_k, const void* W_o,
                                           const int32_t* row_ptr, const int32_t* col_idx, const void* o_s,
                                           const float* lse, const void* d_o, float* d_q, float* d_k, float* d_v,
                                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!o_s || !lse) return fail(HSA_ATTN_ERR_NULL, "o_s and lse are required");
  return backward_impl(desc, q, k, v, U_q, U_k, W_o, row_ptr, col_idx, o_s, lse, d_o, d_q, d_k, d_v,
                       workspace, workspace_bytes, stream);
}
