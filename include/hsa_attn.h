/*
 * hsa_attn.h -- C ABI of the block-sparse + rotary low-rank linear hybrid
 * attention for video diffusion transformers, on AMD gfx950 (MI355X).
 *
 * The operation (SparkDiffusion news article, section 05 "RoLA"; RoLA paper
 * title in the arXiv 2609.23153 listing, "Sources"): a block-sparse softmax
 * branch keeps the high-energy query/key tile interactions, and a low-rank
 * linear-attention branch with rotary position information restores the
 * global context that the sparsification drops; the two are summed.  Raising
 * sparsity from 90% to 97% keeps 3% instead of 10% of the tiles (same article,
 * section 01), which here is a fixed top-k of 64x64 tiles per query-tile row.
 * Reports must state density and block size (Video-Generation-101 handbook
 * chapter on sparse computation, sections 1 and 6), which the CSR and the
 * descriptor carry.
 *
 * Per (b, h) slice, with N valid tokens padded to N_pad = 64*T:
 *   pooling   qbar_a, kbar_a = mean of the valid rows of tile a
 *   scores    sigma_ab = qbar_a . kbar_b
 *   select    M_a = top-k tiles by (sigma desc, index asc) [union {a}]
 *   sparse    O_s,i = softmax over the valid keys of M_a of (scale * q_i . k_j) applied to v
 *   features  phi(x) = elu(x) + 1 of q U_q and k U_k (rank r)
 *   3D RoPE   r dims split 3r/8 : 3r/8 : r/4 over (t, h, w), adjacent pairs,
 *             pair m of an axis block of D dims turns by p_axis * base^(-2m/D)
 *   linear    O_l,i = (rho_i phi_q,i)^T S / (phi_q,i . z),
 *             S = sum_j rho_j phi_k,j v_j^T, z = sum_j phi_k,j over valid j
 *   output    O_i = O_s,i + O_l,i W_o (valid rows), 0 (pad rows)
 *
 * Variant of the linear branch (descriptor field linear_keys): the sums of S
 * and z may instead run, for the queries of tile a, over the valid keys
 * outside the kept tiles M_a only -- the context the sparse branch leaves
 * out (the RoLA section of the SparkDiffusion news article speaks of the
 * linear branch restoring what the sparsification discards; SLA, in the
 * 2026-05-02 survey post on sparse attention for video generation, hands the
 * non-critical weights to linear attention).  A tile whose kept set covers
 * every tile then has O_l = 0.
 *
 * Conventions for every call
 *   - All tensor pointers are DEVICE pointers, owned by the caller; the
 *     library never frees or retains them past the call's stream work.
 *   - Q, K, V, O: [B, H, N_pad, d] row-major, d innermost.  Rows >= N may
 *     hold anything: they are never read as keys, and output rows >= N are
 *     written as zeros.
 *   - U_q, U_k: [H, d, r] row-major; W_o: [H, d, d] row-major (O_l W_o with
 *     O_l a row vector).  Element type: float for in_dtype F32, bf16
 *     otherwise (also for FP8 inputs).
 *   - FP8 inputs: OCP E4M3FN byte codes; *_scale are float [B, H, T], the
 *     value of a code is code * scale of its (b, h, tile).  Scales must be
 *     positive and finite (other values give unspecified outputs) and NULL
 *     for the other dtypes.  The attention calls take FP8 inputs with d = 128
 *     only (HSA_ATTN_ERR_SHAPE otherwise); selection takes any d.  With FP8
 *     inputs both products of the softmax branch run on fp8 operands: the
 *     probabilities of each key tile are rounded to E4M3 after scaling by
 *     that tile's V scale over the largest V scale among the row's kept
 *     tiles, while the softmax statistics stay float32 and unrounded.
 *   - CSR: row_ptr int32 [B*H*T + 1] over the flattened (b, h, a) rows,
 *     starting at 0 and non-decreasing; col_idx int32, each row sorted
 *     ascending.  Output CSR capacity is B*H*T*(topk + force_diag) entries.
 *     In an input CSR, entries outside [0, T) are skipped and a row with no
 *     entries yields O_s = 0 for its queries.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream).  No call synchronises the host or copies device data to
 *     the host, and a call enqueues kernel launches only (no memsets or
 *     copies), so a stream capture of it (a HIP graph) replays the call; with
 *     per-kernel timing on, it also records HIP events.  The library allocates no device memory: scratch space comes
 *     from the caller's workspace of at least hsa_attn_workspace_size()
 *     bytes, 256-byte aligned, which must stay untouched until the stream
 *     work completes.  Calls on different streams with separate workspaces
 *     are independent.
 *   - Every argument is validated before the first launch: a validation
 *     error (NULL, SHAPE, DTYPE, WORKSPACE, CSR) means nothing was enqueued.
 *     HSA_ATTN_ERR_HIP reports a failed launch (earlier kernels of the call
 *     may have been enqueued).  After any non-zero return,
 *     hsa_attn_last_error() (thread-local) holds a message.
 */
#ifndef HSA_ATTN_H
#define HSA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  HSA_ATTN_F32 = 0,      /* float32 */
  HSA_ATTN_BF16 = 1,     /* bfloat16 */
  HSA_ATTN_FP8_E4M3 = 2  /* OCP float8 E4M3FN with per-tile float32 scales */
};

enum {
  HSA_ATTN_OK = 0,
  HSA_ATTN_ERR_NULL = -1,      /* a required pointer is NULL */
  HSA_ATTN_ERR_SHAPE = -2,     /* inconsistent or unsupported sizes */
  HSA_ATTN_ERR_DTYPE = -3,     /* unsupported dtype combination or scales mismatch */
  HSA_ATTN_ERR_WORKSPACE = -4, /* workspace too small or misaligned */
  HSA_ATTN_ERR_CSR = -5,       /* malformed CSR arguments (e.g. only one of a pair given) */
  HSA_ATTN_ERR_HIP = -6        /* a kernel launch failed */
};

enum { /* keys summed by the linear branch (hsa_attn_desc.linear_keys) */
  HSA_ATTN_LINEAR_ALL_KEYS = 0,   /* every valid key (the default) */
  HSA_ATTN_LINEAR_COMPLEMENT = 1  /* per query tile, the valid keys outside its kept tiles */
};

enum { /* which call a workspace size is asked for */
  HSA_ATTN_CALL_BLOCK_SELECT = 0,
  HSA_ATTN_CALL_SPARSE = 1,
  HSA_ATTN_CALL_LINEAR = 2,
  HSA_ATTN_CALL_HYBRID = 3,
  HSA_ATTN_CALL_LINEAR_COMPLEMENT = 4,
  HSA_ATTN_CALL_BACKWARD = 5
};

typedef struct hsa_attn_desc {
  int32_t B, H;             /* batch, heads (>= 1) */
  int32_t N, N_pad;         /* valid tokens; padded length: N_pad % 64 == 0, 0 <= N_pad - N < 64, N >= 1 */
  int32_t d;                /* head dim: 64 or 128 */
  int32_t tile;             /* must be 64 */
  int32_t grid_t, grid_h, grid_w; /* latent grid, grid_t*grid_h*grid_w == N, frame-major raster */
  int32_t topk;             /* tiles kept per row, 1 <= topk <= T */
  int32_t force_diag;       /* 0 or 1: also keep tile a in row a (union) */
  int32_t rank;             /* r: 16, 32 or 64 (multiple of 16) */
  float softmax_scale;      /* > 0, usually 1/sqrt(d) */
  float rope_base;          /* usually 10000 */
  int32_t in_dtype;         /* HSA_ATTN_F32 | HSA_ATTN_BF16 | HSA_ATTN_FP8_E4M3 */
  int32_t out_dtype;        /* F32 with F32 inputs; BF16 with BF16 or FP8 inputs */
  int32_t linear_keys;      /* HSA_ATTN_LINEAR_ALL_KEYS (0) or HSA_ATTN_LINEAR_COMPLEMENT (1),
                               read by hsa_hybrid_attn; the complement needs a mask, so
                               hsa_linear_attn rejects it (HSA_ATTN_ERR_SHAPE; the branch alone
                               is hsa_linear_attn_complement); the complement needs T <= 4096 */
} hsa_attn_desc;

/* Bytes of workspace `call` needs for `desc` (written to *bytes). */
int hsa_attn_workspace_size(const hsa_attn_desc* desc, int call, size_t* bytes);

/* Thread-local message describing the last non-zero return on this thread. */
const char* hsa_attn_last_error(void);

/* Library version string. */
const char* hsa_attn_version(void);

/*
 * Per-kernel timing (a profiling aid, off by default).  While enabled, every
 * kernel the library enqueues is bracketed by HIP events recorded on the same
 * stream, for up to `max_launches` launches per kernel kind; enabling again
 * resets the counts, 0 disables.  hsa_attn_timing_read() waits for the last
 * recorded event and writes, for each kind in HSA_ATTN_KERNEL_* order, the
 * summed milliseconds and the launch count.  Timing adds event records to the
 * stream but no synchronisation to the calls themselves.
 */
enum {
  HSA_ATTN_KERNEL_ROPE = 0,      /* RoPE cos/sin table */
  HSA_ATTN_KERNEL_STREAM = 1,    /* key tile pooling + linear key/value state pass */
  HSA_ATTN_KERNEL_FINALIZE = 2,  /* state reduction, S W_o, readout operands */
  HSA_ATTN_KERNEL_SELECT = 3,    /* query tile pooling, pooled scores, per-row top-k, CSR emission */
  HSA_ATTN_KERNEL_UNUSED4 = 4,   /* no kernel is timed under this kind */
  HSA_ATTN_KERNEL_ATTEND = 5,    /* block-sparse flash attention + linear readout */
  HSA_ATTN_KERNEL_QUANT = 6,     /* per-row FP8 quantisation of activations */
  HSA_ATTN_KERNEL_PROJ = 7,      /* W8A8 FP8 QKV projection with fused output quantisation */
  HSA_ATTN_KERNEL_COMPL = 8,     /* linear branch over the complement of the kept tiles */
  HSA_ATTN_KERNEL_BWD_LINEAR = 9,  /* backward: linear branch (query side, sums, key side) */
  HSA_ATTN_KERNEL_BWD_SPARSE = 10, /* backward: transposed mask, sparse dQ and dK/dV */
  HSA_ATTN_KERNEL_KINDS = 11
};
int hsa_attn_timing_enable(int max_launches);
int hsa_attn_timing_read(double* ms_out, int32_t* launches_out);

/*
 * Read-rate calibration (a measurement aid, not part of the attention): reads
 * `bytes` (a positive multiple of 16) from the device buffer `buf` once with
 * 16-byte loads and writes one XOR-folded word per thread into the device
 * array `sink` (at least HSA_ATTN_READ_SINK_WORDS words, caller-owned).  Its
 * duration gives the read rate a plain streaming kernel reaches from this
 * GPU's memory, the practical ceiling for the streaming pass over K and V.
 * Asynchronous on `stream`; errors: NULL, SHAPE (nothing launched), HIP.
 */
#define HSA_ATTN_READ_SINK_WORDS (2048 * 256)
int hsa_attn_read_calibrate(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words, void* stream);

/*
 * Tile selection (SparkDiffusion news article, section 05: the sparse branch
 * keeps the high-energy query/key tile interactions; section 01: 90% / 97% of
 * the tiles are skipped, here a fixed top-k per query-tile row).  Mean-pool Q
 * and K per 64-token tile (float64 sums of the valid rows), score every
 * (query tile, key tile) pair by the dot product of the means, keep the top-k
 * key tiles of every row (ties: lower index first; plus the diagonal tile if
 * force_diag) and emit them as CSR.  The kept set is the one the float64
 * scores give: scores are formed on the matrix cores from bf16 hi + lo parts
 * of the means with a rigorous error bound, and the tiles whose score lies
 * within that bound of the k-th one are ranked again by their float64 scores.
 *   q, k: [B, H, N_pad, d] device, in_dtype; q_scale, k_scale: FP8 tile scales.
 *   row_ptr [B*H*T + 1], col_idx [B*H*T*(topk+force_diag)]: outputs.
 *   qbar_out, kbar_out: optional float64 [B, H, T, d] tile means (NULL to skip).
 *   Workspace: HSA_ATTN_CALL_BLOCK_SELECT.  Errors as for every call.
 */
int hsa_block_select(const hsa_attn_desc* desc, const void* q, const void* k,
                     const float* q_scale, const float* k_scale,
                     int32_t* row_ptr, int32_t* col_idx,
                     double* qbar_out, double* kbar_out,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Block-sparse softmax branch on a given CSR (SparkDiffusion news article,
 * section 05: exact softmax attention on the kept high-energy tiles; section
 * 01: 3% of the 64x64 tiles kept at 97% sparsity): for each query tile, flash
 * attention over the kept key tiles with float32 softmax statistics.  With
 * FP8 inputs the workspace holds V transposed per tile (B*H*N_pad*d bytes);
 * the other dtypes need none.
 *   o_sparse: [B, H, N_pad, d] in out_dtype (rows >= N zero).
 *   lse_out: optional float [B, H, N_pad] natural-log sum of exp(scale*q.k)
 *   over the kept valid keys (NULL to skip; rows >= N undefined).
 */
int hsa_sparse_attn(const hsa_attn_desc* desc, const void* q, const void* k, const void* v,
                    const float* q_scale, const float* k_scale, const float* v_scale,
                    const int32_t* row_ptr, const int32_t* col_idx,
                    void* o_sparse, float* lse_out,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Rotary low-rank linear branch alone (SparkDiffusion news article, section
 * 05: a low-rank linear-attention branch carrying rotary position information
 * restores the global context), already multiplied by W_o:
 *   o_lin = O_l W_o, [B, H, N_pad, d] in out_dtype (rows >= N zero).
 * The key/value state is reduced in a fixed order (bitwise reproducible).
 */
int hsa_linear_attn(const hsa_attn_desc* desc, const void* q, const void* k, const void* v,
                    const float* q_scale, const float* k_scale, const float* v_scale,
                    const void* U_q, const void* U_k, const void* W_o,
                    void* o_lin, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The linear branch over the complement of a given mask (SparkDiffusion news
 * article, section 05: the linear branch restores what the sparsification
 * discards; SLA in the 2026-05-02 survey post, item 1), alone, already
 * multiplied by W_o: for the queries of tile a, the sums of S and z run over
 * the valid keys outside the tiles of CSR row a (entries outside [0, T) and
 * repeats name no extra tile; a row naming every tile gives O_l = 0).  The
 * descriptor's linear_keys is not read; T <= 4096.  The workspace size is the
 * one of HSA_ATTN_CALL_LINEAR_COMPLEMENT.
 *   o_lin: [B, H, N_pad, d] in out_dtype (rows >= N zero).
 */
int hsa_linear_attn_complement(const hsa_attn_desc* desc, const void* q, const void* k, const void* v,
                               const float* q_scale, const float* k_scale, const float* v_scale,
                               const void* U_q, const void* U_k, const void* W_o,
                               const int32_t* row_ptr, const int32_t* col_idx, void* o_lin,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * The whole hybrid (SparkDiffusion news article, section 05: the block-sparse
 * softmax branch and the rotary low-rank linear branch, summed; section 01:
 * the top-k tile budget per row): O = O_s + O_l W_o, selection included.
 *   With linear_keys = HSA_ATTN_LINEAR_COMPLEMENT, O_l of the queries of tile
 *   a sums over the valid keys outside the tiles of CSR row a (entries
 *   outside [0, T) and repeats name no extra tile); the workspace then also
 *   holds one r x d state per key tile (B*H*T*d*32*ceil(r/32) elements of
 *   the parameter type), and the kept tiles' states are subtracted from the
 *   full state, or, when a row keeps more than half of the tiles, the others'
 *   states are summed directly.
 *   row_ptr_in / col_idx_in: if both non-NULL, use this mask and skip
 *   selection; if both NULL, select as hsa_block_select does.
 *   row_ptr_out / col_idx_out: if both non-NULL (and no mask was given),
 *   also export the selected CSR; both NULL to skip.
 *   o: [B, H, N_pad, d] in out_dtype.
 */
int hsa_hybrid_attn(const hsa_attn_desc* desc, const void* q, const void* k, const void* v,
                    const float* q_scale, const float* k_scale, const float* v_scale,
                    const void* U_q, const void* U_k, const void* W_o,
                    const int32_t* row_ptr_in, const int32_t* col_idx_in,
                    int32_t* row_ptr_out, int32_t* col_idx_out,
                    void* o, void* workspace, size_t workspace_bytes, void* stream);

/*
 * hsa_hybrid_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same call and result, with the scratch taken from a static device array
 * of HSA_ATTN_STATIC_SCRATCH_BYTES (256 MiB) that the library holds on every
 * GPU it runs on until the process ends.  A call whose workspace would exceed
 * it returns HSA_ATTN_ERR_WORKSPACE before anything is enqueued (the
 * workspace size of HSA_ATTN_CALL_HYBRID says how much a call needs; the
 * 720P bf16 call needs ~140 MiB, FP8 at 720P ~510 MiB and is rejected).
 * Every call on one GPU shares that array, so calls that overlap in time on
 * one GPU (different streams, or threads) race and must be serialised by the
 * caller; nothing in the array needs to start at zero.  The first call on a
 * device takes the array's address there (hipGetSymbolAddress); no call
 * allocates.
 */
#define HSA_ATTN_STATIC_SCRATCH_BYTES ((size_t)256 << 20)
int hsa_hybrid_attn_noalloc(const hsa_attn_desc* desc, const void* q, const void* k, const void* v,
                            const float* q_scale, const float* k_scale, const float* v_scale,
                            const void* U_q, const void* U_k, const void* W_o,
                            const int32_t* row_ptr_in, const int32_t* col_idx_in,
                            int32_t* row_ptr_out, int32_t* col_idx_out, void* o, void* stream);

/*
 * Backward pass of the hybrid (all-keys linear branch) on the forward's mask
 * (the pages adapt the dense model to the sparse RoLA structure with a short
 * sparse warm-up, which trains through the operator: SparkDiffusion news
 * article, section 05; project blog, "A simple staging principle", item 1):
 * the gradients of L with respect to Q, K and V given dL/dO = d_o, with the
 * tile selection held fixed (it is piecewise constant in the inputs).  The
 * forward's linear state and the sparse branch's output and log-sum-exp are
 * recomputed from q, k, v, so nothing of the forward call is needed besides
 * its mask.  Sparse branch: P = softmax(scale q k^T) over the kept keys,
 * dS = P * (dO v^T - D) with D_i = dO_i . O_s,i; dq += scale dS k,
 * dk += scale dS^T q, dv += P^T dO.  Linear branch: the chain rule through
 * O_l = num / den (see hsa_linear_attn), S and z.
 *   q, k, v: [B, H, N_pad, d] float32 or bf16 (HSA_ATTN_ERR_DTYPE for FP8);
 *   U_q, U_k, W_o as for the forward; row_ptr / col_idx: the forward's CSR
 *   (entries outside [0, T) are skipped; rows with repeated entries, or with
 *   more than topk + force_diag entries in [0, T), are outside this call's
 *   domain: the transposed mask it builds holds B*H*T*(topk + force_diag)
 *   entries, so set topk to the longest row of a mask not made by selection);
 *   d_o: [B, H, N_pad, d] in the input type (rows >= N are ignored).
 *   d_q, d_k, d_v: float32 [B, H, N_pad, d], written in full (rows >= N zero).
 *   desc->linear_keys must be HSA_ATTN_LINEAR_ALL_KEYS (HSA_ATTN_ERR_SHAPE
 *   otherwise).  Workspace: HSA_ATTN_CALL_BACKWARD.
 */
int hsa_hybrid_attn_backward(const hsa_attn_desc* desc, const void* q, const void* k, const void* v,
                             const void* U_q, const void* U_k, const void* W_o,
                             const int32_t* row_ptr, const int32_t* col_idx, const void* d_o,
                             float* d_q, float* d_k, float* d_v,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Training forward: hsa_hybrid_attn (all-keys linear branch, float32 or bf16
 * inputs) that also saves what the backward needs from it, as FlashAttention
 * saves its log-sum-exp, so that hsa_hybrid_attn_backward_saved can skip the
 * sparse recompute (one attention pass).  Same passages as the backward: the
 * sparse warm-up trains through the operator (SparkDiffusion news article,
 * section 05; project blog, "A simple staging principle", item 1).
 *   Arguments as for hsa_hybrid_attn (no scales: FP8 inputs and the
 *   complement variant give HSA_ATTN_ERR_DTYPE / HSA_ATTN_ERR_SHAPE, and topk
 *   must lie in [1, T] also with a given mask, as for the backward), plus
 *   o_s: [B, H, N_pad, d] in out_dtype, the sparse branch's output O_s alone
 *   (rows >= N zero), bitwise what hsa_sparse_attn writes on the same mask;
 *   lse: float [B, H, N_pad], its natural-log log-sum-exp (rows >= N
 *   undefined), as hsa_sparse_attn's lse.  Both required (HSA_ATTN_ERR_NULL).
 *   o is bitwise what hsa_hybrid_attn writes.  Workspace: HSA_ATTN_CALL_HYBRID.
 */
int hsa_hybrid_attn_train(const hsa_attn_desc* desc, const void* q, const void* k, const void* v,
                          const void* U_q, const void* U_k, const void* W_o,
                          const int32_t* row_ptr_in, const int32_t* col_idx_in,
                          int32_t* row_ptr_out, int32_t* col_idx_out, void* o, void* o_s, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * hsa_hybrid_attn_backward with the sparse branch's output and log-sum-exp
 * taken from hsa_hybrid_attn_train (o_s, lse: as that call wrote them, for
 * the same inputs and mask) instead of recomputed: the same gradients, bit
 * for bit, without one attention pass.  o_s and lse are required
 * (HSA_ATTN_ERR_NULL); everything else as for hsa_hybrid_attn_backward.
 * Workspace: HSA_ATTN_CALL_BACKWARD.
 */
int hsa_hybrid_attn_backward_saved(const hsa_attn_desc* desc, const void* q, const void* k, const void* v,
                                   const void* U_q, const void* U_k, const void* W_o,
                                   const int32_t* row_ptr, const int32_t* col_idx, const void* o_s,
                                   const float* lse, const void* d_o, float* d_q, float* d_k, float* d_v,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * W8A8 FP8 projections in front of the attention (SparkDiffusion news
 * article, section 07: the linear projections are quantised to W8A8 FP8
 * E4M3, with activation scaling and type conversion fused into the kernels).
 *
 * Per-row FP8 quantisation of activations (the A8 half):
 *   x: bfloat16 [M, C] row-major, device.  C a multiple of 8 (HSA_ATTN_ERR_SHAPE
 *   otherwise), M >= 0.
 *   codes_out: E4M3FN bytes [M, C]; scales_out: float [M], device, caller-owned.
 *   Row m: s = max|x_m| / 448 (1 for an all-zero row), code = round-to-nearest-
 *   even(x / s); both divisions correctly rounded float32.
 */
int hsa_quantize_rows_fp8(const void* x, int64_t M, int64_t C, void* codes_out, float* scales_out,
                          void* stream);

/*
 * QKV projection on the FP8 matrix cores, writing the attention's FP8 inputs:
 *   Y[m, j] = s_x[m] s_w[j] sum_c x8[m, c] w8[j, c],  m = b N_pad + n,
 *   j = (t H + h) d + e for tensor t (0 = q, 1 = k, 2 = v), head h, dim e;
 *   then, per (tensor, b, h, 64-token tile): s = max|Y| / 448 over the tile's
 *   64 x d values (1 if all zero) and code = round-to-nearest-even(Y / s),
 *   taken from the float32 accumulators (multiplied by the float32
 *   reciprocal of s).
 *   x_codes: E4M3FN [B*N_pad, C], x_scales: float [B*N_pad] (as written by
 *   hsa_quantize_rows_fp8; pad rows should be zero).
 *   w_codes: E4M3FN [3*H*d, C] (row j = output column j), w_scales: float [3*H*d].
 *   q, k, v: E4M3FN [B, H, N_pad, d]; q_scales, k_scales, v_scales: float
 *   [B, H, N_pad/64] -- exactly the FP8 inputs of hsa_hybrid_attn.
 *   Requires d = 128, C a multiple of 128 (128 <= C, 256*C < 2^31),
 *   N_pad a multiple of 64, B, H >= 1 (HSA_ATTN_ERR_SHAPE otherwise).  All
 *   pointers device, caller-owned; nothing is allocated.
 */
int hsa_qkv_proj_fp8(const void* x_codes, const float* x_scales, const void* w_codes, const float* w_scales,
                     int32_t B, int32_t N_pad, int32_t C, int32_t H, int32_t d,
                     void* q, void* k, void* v, float* q_scales, float* k_scales, float* v_scales,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HSA_ATTN_H */
