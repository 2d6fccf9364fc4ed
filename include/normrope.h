/*
 * normrope.h -- C ABI of libnormrope.so: single-pass fused RMSNorm and
 * LayerNorm (forward and backward), in-place interleaved RoPE (forward and
 * inverse), their fusions (RMSNorm -> RoPE, LayerNorm -> GeLU) and RMSNorm
 * folded into the following linear layer, for AMD Instinct MI355X (gfx950).
 *
 * The operations follow "Helios 性能优化全解析" (hncyxsy.com), sections
 * 内核一 FlashNorm and 内核二 FlashRoPE, and the fused LayerNorm example of
 * "LLM层的优化算子" (apxml.com), section 编写定制融合算子.
 *
 * Conventions for every call below
 *   - Pointers are DEVICE pointers unless stated otherwise.  The caller owns
 *     every buffer; the library allocates nothing and keeps no pointer after
 *     the call returns.
 *   - Tensors are dense and row-major: a norm input is [rows][n] with row
 *     stride n.  x, y, dy, dx, w, gamma and beta share the dtype `dt`.
 *     Per-row statistics, dw / dgamma / dbeta and RoPE tables are fp32.
 *   - All arithmetic is fp32; each stored bf16 or fp16 value is rounded
 *     once, to nearest even.
 *   - Work is queued on `stream` (a hipStream_t; NULL = default stream) and
 *     the call returns without waiting for it.
 *   - Arguments are checked on the host before anything is queued.  On any
 *     error the call returns a non-zero nr_status_t and queues nothing,
 *     except NR_ERR_HIP, which reports a failed launch (see
 *     nr_last_hip_error).  rows == 0 (or tokens == 0) is a valid no-op.
 *   - Any alignment is accepted by the norm and RoPE calls.  Rows whose
 *     start is 16-byte aligned and whose byte length is a multiple of 16
 *     take the 128-bit load path; other shapes take an element-wise path in
 *     the same kernels.  (The linear-layer calls need 16-byte alignment.)
 *   - An output may be the very same buffer as an input of the same shape
 *     (in place: y == x, dx == dy or dx == x); no other output, and no
 *     workspace, may share a byte with any operand of the call (weights, row
 *     statistics, tables, column gradients included), else NR_ERR_ALIAS.
 *     The backward kernels read the row statistics through the scalar cache,
 *     which writes to other buffers do not update.
 *   - Backward results are bitwise reproducible: for a given shape every
 *     summation order is fixed (no atomics), whatever the device.
 *   - Thread safety: calls may be made from several host threads; the only
 *     shared state is the tuning table set by nr_tune and the scratch array
 *     of rmsnorm_bwd_noalloc.
 */
#ifndef NORMROPE_H
#define NORMROPE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of the row / token tensors and their weights.  Arithmetic is
 * fp32 whatever the storage type; each stored result is rounded once, to
 * nearest even. */
typedef enum {
  NR_F32 = 0,
  NR_BF16 = 1,
  NR_F16 = 2, /* IEEE binary16 */
  /* not dtypes: they make every int a value of the type, so an unknown code
     passed in is rejected (NR_ERR_DTYPE) rather than out of the type's range */
  NR_DTYPE_RANGE_MIN_ = -0x7fffffff - 1,
  NR_DTYPE_RANGE_MAX_ = 0x7fffffff
} nr_dtype_t;

typedef enum {
  NR_OK = 0,
  NR_ERR_NULLPTR = 1,       /* a required pointer is NULL */
  NR_ERR_SHAPE = 2,         /* negative size, n < 1, odd head_dim, bad grid */
  NR_ERR_DTYPE = 3,         /* dt is not NR_F32 / NR_BF16 / NR_F16 */
  NR_ERR_UNSUPPORTED_N = 4, /* n (or a head's size) beyond the on-chip limit */
  NR_ERR_WORKSPACE = 5,     /* workspace missing, too small or not 16-byte aligned */
  NR_ERR_HIP = 6,           /* the HIP runtime refused a launch */
  NR_ERR_ALIAS = 7,         /* an output partially overlaps an input */
  NR_ERR_TUNE = 8,          /* unknown tuning key or value */
  /* not statuses: every int is a value of the type (nr_status_str of an
     unknown code returns a description saying so) */
  NR_STATUS_RANGE_MIN_ = -0x7fffffff - 1,
  NR_STATUS_RANGE_MAX_ = 0x7fffffff
} nr_status_t;

/* Largest row length the norm kernels accept: 65536 (bf16, fp16), 32768 (fp32). */
int64_t nr_norm_n_max(nr_dtype_t dt); /* host only */

/*
 * rmsnorm_fwd -- Helios 性能优化全解析, 内核一 FlashNorm.
 *   for each row i:  r_i = 1 / sqrt(mean_j x_ij^2 + eps)
 *                    y_ij = (x_ij * r_i) * w'_j
 *   with w'_j = w_j, or 1 + w_j when gemma_offset != 0 (the Gemma variant),
 *   or 1 when w is NULL.  inv_rms[i] = r_i is stored when inv_rms != NULL
 *   (it is what rmsnorm_bwd reads).
 *   x [rows][n], y [rows][n] (may be x), w [n] or NULL, inv_rms [rows] fp32
 *   or NULL.
 */
nr_status_t rmsnorm_fwd(nr_dtype_t dt, const void* x, const void* w, void* y,
                        float* inv_rms, int64_t rows, int64_t n, float eps,
                        int gemma_offset, void* stream);

/*
 * rmsnorm_bwd -- backward of rmsnorm_fwd; reads the cached inv_rms instead
 * of recomputing it (内核一 FlashNorm: the backward reuses the forward's
 * per-row cache).
 *   xhat = x * r, g = dy * w', c_i = mean_j g_ij xhat_ij
 *   dx_ij = r_i (g_ij - xhat_ij c_i)            -> dx [rows][n] (may be dy)
 *   dw_j  = sum_i dy_ij xhat_ij (fp32)          -> dw [n] or NULL (not formed)
 *   dw is a two-stage fixed-order reduction through `workspace` (device,
 *   16-byte aligned, at least nr_bwd_workspace_bytes(rows, n, 0) bytes).
 *   Rows of more than 16384 elements take two passes over the rows (a row
 *   reduction first, then dx and the column partials by column slices) and
 *   keep two fp32 terms per row in the workspace, so for them it is
 *   required even when dw is NULL; otherwise it may be NULL when dw is.
 *   Exception: bf16 / fp16 rows of up to 32768 elements with dy, x, dx and
 *   w 16-byte aligned and n a multiple of 8 take one pass here (not in
 *   rmsnorm_rope_bwd or the LayerNorm backwards).
 *   The workspace is scratch: its content on entry does not matter and is
 *   overwritten.
 */
nr_status_t rmsnorm_bwd(nr_dtype_t dt, const void* dy, const void* x,
                        const void* w, const float* inv_rms, void* dx,
                        float* dw, int64_t rows, int64_t n, int gemma_offset,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * rmsnorm_bwd_noalloc -- rmsnorm_bwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same operation, arguments and kernels without the
 * workspace arguments.  The partial rows go to a scratch array the library
 * holds in device memory, one copy per GPU, for as long as it is loaded.
 * Its limit is NR_NOALLOC_SCRATCH_BYTES: a call whose
 * nr_bwd_workspace_bytes(rows, n, 0) exceeds it (only batches of millions
 * of rows longer than 16384 elements can) returns NR_ERR_WORKSPACE and
 * queues nothing.
 * The call allocates nothing.  Its first call on a device looks the array's
 * address up on that device (outside any graph capture, so make one call
 * before capturing); a failed lookup returns NR_ERR_HIP.
 * Every call on one GPU shares that GPU's array: calls that may run at the
 * same time on one GPU (different streams without ordering between them)
 * race on it and must not be made.  Nothing in the array needs to start at
 * zero; it keeps the last call's contents.
 */
#define NR_NOALLOC_SCRATCH_BYTES (32u << 20)
nr_status_t rmsnorm_bwd_noalloc(nr_dtype_t dt, const void* dy, const void* x,
                                const void* w, const float* inv_rms, void* dx,
                                float* dw, int64_t rows, int64_t n,
                                int gemma_offset, void* stream);

/*
 * layernorm_fwd -- 内核一 FlashNorm (mean, variance and scale in one read of
 * the row) with the formula of 编写定制融合算子 (biased variance, eps inside
 * the root, then weight and bias):
 *   mu_i = mean_j x_ij, var_i = mean_j (x_ij - mu_i)^2, r_i = 1/sqrt(var_i + eps)
 *   y_ij = (x_ij - mu_i) r_i gamma_j + beta_j    (gamma NULL -> 1, beta NULL -> 0)
 *   mean[i] = mu_i and rstd[i] = r_i are stored when non-NULL (fp32 [rows]).
 */
nr_status_t layernorm_fwd(nr_dtype_t dt, const void* x, const void* gamma,
                          const void* beta, void* y, float* mean, float* rstd,
                          int64_t rows, int64_t n, float eps, void* stream);

/*
 * layernorm_bwd -- backward of layernorm_fwd from the cached mean and rstd.
 *   xhat = (x - mu) r, g = dy gamma, a_i = mean_j g, b_i = mean_j g xhat
 *   dx = r (g - a - xhat b)                      -> dx [rows][n] (may be dy)
 *   dgamma_j = sum_i dy xhat, dbeta_j = sum_i dy -> fp32 [n] each, or NULL
 *   workspace: at least nr_bwd_workspace_bytes(rows, n, 1) bytes, under
 *   the same rules as rmsnorm_bwd.
 */
nr_status_t layernorm_bwd(nr_dtype_t dt, const void* dy, const void* x,
                          const void* gamma, const float* mean,
                          const float* rstd, void* dx, float* dgamma,
                          float* dbeta, int64_t rows, int64_t n,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * rope_interleaved_apply -- Helios 性能优化全解析, 内核二 FlashRoPE.
 *   x is [batch][tokens][heads][head_dim] with element strides stride_batch,
 *   stride_token, stride_head (the head_dim axis is contiguous).  For each
 *   pair i < head_dim/2 of each head vector, with (a, b) = (x[2i], x[2i+1]),
 *   c = cos_tab[t][i], s = sin_tab[t][i] and sigma = -1 if inverse else +1:
 *       x[2i]   = a c - b (sigma s)
 *       x[2i+1] = a (sigma s) + b c
 *   written IN PLACE.  The inverse is also the backward (the rotation's
 *   transpose).  Tables are fp32 [tokens][head_dim/2], shared by all heads
 *   and batches; build them with rope_table_1d / rope_table_3d or supply
 *   your own.  head_dim must be even.  Distinct (batch, token, head) vectors
 *   must not share elements, else NR_ERR_ALIAS: with the axes of size > 1
 *   ordered by stride, each stride must be at least the span of the axes
 *   inside it, starting from head_dim (so no stride 0 on such an axis;
 *   transposed layouts such as [batch][heads][tokens] pass).  A token's
 *   heads must span less than 1 GiB
 *   ((heads-1)*stride_head + head_dim elements), else NR_ERR_UNSUPPORTED_N.
 */
nr_status_t rope_interleaved_apply(nr_dtype_t dt, void* x, const float* cos_tab,
                                   const float* sin_tab, int64_t batch,
                                   int64_t tokens, int64_t heads,
                                   int64_t head_dim, int64_t stride_batch,
                                   int64_t stride_token, int64_t stride_head,
                                   int inverse, void* stream);

/*
 * rope_table_1d -- cos/sin table for 1-D positions pos0 .. pos0+tokens-1:
 *   angle(t, i) = (pos0 + t) * theta^(-2i/head_dim), i < head_dim/2,
 *   computed in double, cos and sin rounded once to fp32.
 *   cos_tab, sin_tab: device fp32 [tokens][head_dim/2].
 */
nr_status_t rope_table_1d(float* cos_tab, float* sin_tab, int64_t tokens,
                          int64_t head_dim, int64_t pos0, double theta,
                          void* stream);

/*
 * rope_table_3d -- cos/sin table for a frames x height x width token grid,
 * tokens ordered frame-major, then row, then column.  The head_dim/2 =
 * pairs_t + pairs_h + pairs_w pairs are split into consecutive blocks that
 * follow the frame, row and column index; pair j of a block of P pairs uses
 * frequency theta^(-2j/(2P)).  Device fp32 [frames*height*width][head_dim/2].
 */
nr_status_t rope_table_3d(float* cos_tab, float* sin_tab, int64_t frames,
                          int64_t height, int64_t width, int64_t pairs_t,
                          int64_t pairs_h, int64_t pairs_w, double theta,
                          void* stream);

/*
 * rmsnorm_rope_fwd -- rmsnorm_fwd followed by interleaved RoPE on its output,
 * fused into one pass: each row is read once and written once, rotated
 * before its single rounding (the two operations of Helios 性能优化全解析,
 * 内核一 FlashNorm and 内核二 FlashRoPE, which the write-up measures
 * together).  A row of n = (heads in the row) x head_dim elements is
 * normalised as in rmsnorm_fwd, then each head vector's pair i is rotated by
 * cos_tab[tok][i], sin_tab[tok][i], tok = row / rows_per_token (1 when a row
 * is a whole token; heads when each head is normalised on its own).  Tables
 * are fp32 [rows / rows_per_token][head_dim / 2].  y may be x; inv_rms as in
 * rmsnorm_fwd.
 */
nr_status_t rmsnorm_rope_fwd(nr_dtype_t dt, const void* x, const void* w,
                             void* y, float* inv_rms, const float* cos_tab,
                             const float* sin_tab, int64_t rows, int64_t n,
                             int64_t head_dim, int64_t rows_per_token,
                             float eps, int gemma_offset, void* stream);

/*
 * rmsnorm_rope_bwd -- backward of rmsnorm_rope_fwd: dout (the gradient of
 * the rotated output) is rotated back by the same angles (sin negated) in
 * registers and fed to the rmsnorm_bwd arithmetic; dx [rows][n] (may be
 * dout), dw [n] fp32 or NULL.  Workspace rules as for rmsnorm_bwd, size
 * nr_bwd_workspace_bytes(rows, n, 2).
 */
nr_status_t rmsnorm_rope_bwd(nr_dtype_t dt, const void* dout, const void* x,
                             const void* w, const float* inv_rms,
                             const float* cos_tab, const float* sin_tab,
                             void* dx, float* dw, int64_t rows, int64_t n,
                             int64_t head_dim, int64_t rows_per_token,
                             int gemma_offset, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * layernorm_gelu_fwd -- layernorm_fwd with the tanh-approximated GeLU applied
 * to its output in the same pass, the fused LayerNorm + GeLU of "LLM层的优化
 * 算子", section 编写定制融合算子:
 *   y = gelu(a), a = (x - mu) r gamma + beta,
 *   gelu(v) = v/2 (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))).
 * mean and rstd are stored as in layernorm_fwd (the backward recomputes a).
 */
nr_status_t layernorm_gelu_fwd(nr_dtype_t dt, const void* x, const void* gamma,
                               const void* beta, void* y, float* mean,
                               float* rstd, int64_t rows, int64_t n, float eps,
                               void* stream);

/*
 * layernorm_gelu_bwd -- backward of layernorm_gelu_fwd: the pre-activation a
 * is recomputed from x, the cached mean / rstd, gamma and beta; dy = dout *
 * gelu'(a) feeds the layernorm_bwd arithmetic.  Outputs and workspace as
 * for layernorm_bwd (nr_bwd_workspace_bytes(rows, n, 1)).
 */
nr_status_t layernorm_gelu_bwd(nr_dtype_t dt, const void* dout, const void* x,
                               const void* gamma, const void* beta,
                               const float* mean, const float* rstd, void* dx,
                               float* dgamma, float* dbeta, int64_t rows,
                               int64_t n, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * rmsnorm_linear_fwd -- RMSNorm folded into the linear layer that consumes
 * it: the norm -> linear fusion of "HY-Motion 1.0性能优化" (section 3.1
 * 算子融合与计算图优化: the normalisation merged with the following matrix
 * multiplication, so the intermediate is neither stored nor re-read) and of
 * "Janus-Pro-7B模型推理加速实战" (section 4.1 融合的LayerNorm与线性层内核),
 * with the RMSNorm of Helios 性能优化全解析, 内核一 FlashNorm as the norm:
 *   r_m = 1/sqrt(mean_k x[m][k]^2 + eps)            -> inv_rms [M] (or NULL)
 *   out[m][n] = r_m sum_k x[m][k] w'_k W[n][k]      -> out [M][N]
 * i.e. out = rmsnorm_fwd(x, w_norm) W^T with W [N][K] row-major (the layout
 * of a linear layer's weight), w'_k = w_k, 1 + w_k (gemma_offset) or 1
 * (w_norm NULL).  bf16 only (NR_BF16): x enters the bf16 matrix cores
 * exactly, w'_k W[n][k] is rounded once to bf16, accumulation is fp32 and
 * out is rounded once.  Forward only.
 * Shapes: K a multiple of 64 (at most 65536), N a multiple of 128, any M;
 * x, W, out and w_norm 16-byte aligned (else NR_ERR_SHAPE); out may not
 * overlap x or W.
 * Workspace: when N is a multiple of 256 the call first computes
 * the row statistics (into inv_rms, or the workspace's first ceil(4 M /
 * 256) 256 bytes when inv_rms is NULL) and, with a norm weight, writes the
 * folded weight w'_k W[n][k] (N K bf16) into the workspace after them;
 * nr_rmsnorm_linear_workspace_bytes gives the size to pass (0 when none is
 * needed).  A workspace that is NULL, smaller than needed or not 16-byte
 * aligned when one is needed is NR_ERR_WORKSPACE; one overlapping an operand
 * is NR_ERR_ALIAS.  Its contents on return are unspecified.
 */
nr_status_t rmsnorm_linear_fwd(nr_dtype_t dt, const void* x, const void* w_norm,
                               const void* W, void* out, float* inv_rms,
                               int64_t M, int64_t N, int64_t K, float eps,
                               int gemma_offset, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * layernorm_linear_fwd -- LayerNorm folded into the linear layer that
 * consumes it ("HY-Motion 1.0性能优化", section 3.1 算子融合与计算图优化:
 * LayerNorm's mean and variance merged with the following matrix
 * multiplication, so the normalised activation is neither stored nor
 * re-read; "Janus-Pro-7B模型推理加速实战", section 4.1
 * 融合的LayerNorm与线性层内核):
 *   mu_m = mean_k x[m][k], r_m = 1/sqrt(mean_k (x[m][k] - mu_m)^2 + eps)
 *                                             -> mean, rstd [M] (or NULL)
 *   out[m][n] = sum_k ((x[m][k] - mu_m) r_m gamma_k + beta_k) W[n][k]
 *                                             -> out [M][N]
 * i.e. out = layernorm_fwd(x, gamma, beta) W^T with W [N][K] row-major;
 * gamma NULL -> 1, beta NULL -> 0.  bf16 only (NR_BF16).  It is evaluated
 * as r_m (sum_k x[m][k] Wf[n][k] - mu_m c_n) + d_n: x enters the bf16
 * matrix cores exactly, Wf = gamma_k W[n][k] rounded once to bf16,
 * c_n = sum_k Wf[n][k] and d_n = sum_k beta_k W[n][k] in fp32, fp32
 * accumulation, out rounded once.  (The mean is removed after the product:
 * for rows whose mean is large against their spread, the fp32 accumulation
 * of the uncentred product bounds the accuracy.)  Forward only.
 * Shapes: K a multiple of 64 (at most 65536), N a multiple of 256 (at most
 * 2^22), any M; x, W, out, gamma and beta 16-byte aligned (else
 * NR_ERR_SHAPE); out may not overlap x or W.
 * Workspace: nr_layernorm_linear_workspace_bytes(M, N, K, gamma != NULL)
 * bytes, 16-byte aligned and apart from every operand (else
 * NR_ERR_WORKSPACE / NR_ERR_ALIAS); it takes the row statistics when mean
 * or rstd is NULL, the column terms and the folded weight.  Its contents on
 * return are unspecified.
 */
nr_status_t layernorm_linear_fwd(nr_dtype_t dt, const void* x, const void* gamma,
                                 const void* beta, const void* W, void* out,
                                 float* mean, float* rstd, int64_t M, int64_t N,
                                 int64_t K, float eps, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Workspace bytes layernorm_linear_fwd needs at this shape (has_gamma: a
 * gamma will be passed); 0 for a shape it does not take.  Host only. */
size_t nr_layernorm_linear_workspace_bytes(int64_t M, int64_t N, int64_t K,
                                           int has_gamma);

/* Workspace bytes rmsnorm_linear_fwd may need at this shape (has_weight: a
 * norm weight is passed): on the large-tile path ceil(4 M / 256) 256 for
 * the row statistics plus N K 2 for the folded weight, else 0.  Host only;
 * a pure function of its arguments and the current tuning table. */
size_t nr_rmsnorm_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int has_weight);

/*
 * rmsnorm_linear_fold_weight -- the folded weight of rmsnorm_linear_fwd on
 * its own: W_folded[n][k] = bf16(W[n][k] w'_k), w'_k = w_k or 1 + w_k
 * (gemma_offset), one rounding.  For callers whose weights do not change
 * between calls: rmsnorm_linear_fwd(x, NULL, W_folded, ...) then gives the
 * same output, bit for bit, as rmsnorm_linear_fwd(x, w_norm, W, ...) without
 * folding the weight again (and needs no workspace room for it).  bf16 only; K a multiple of 8 (at most 65536), N at
 * most 2^22; all three pointers 16-byte aligned; W_folded may be W (in
 * place) but may not partly overlap it or overlap w_norm.
 */
nr_status_t rmsnorm_linear_fold_weight(nr_dtype_t dt, const void* w_norm, const void* W,
                                       void* W_folded, int64_t N, int64_t K,
                                       int gemma_offset, void* stream);

/* Workspace bytes a backward call needs for dw / dgamma / dbeta at this
 * shape, for any dtype: op = 0 rmsnorm_bwd, 1 layernorm_bwd or
 * layernorm_gelu_bwd, 2 rmsnorm_rope_bwd (0 for any other op).  An upper
 * bound: some (dtype, n) use fewer workgroups and so less.  Host only; a
 * pure function of its arguments and the current tuning table. */
size_t nr_bwd_workspace_bytes(int64_t rows, int64_t n, int op);

/* Static description of a status code.  Host only. */
const char* nr_status_str(nr_status_t s);

/* hipError_t of the last NR_ERR_HIP seen by the calling thread (0 if none). */
int nr_last_hip_error(void);

/*
 * nr_tune -- override one launch-shape choice (for tuning sweeps; results
 * stay within the same tolerances, but the backward's summation order, and
 * so its exact bits, depend on the shape).  value 0 restores the automatic
 * choice.  Keys: "fwd_w", "fwd_k", "fwd_r", "fwd_j", "bwd_w", "bwd_k",
 * "bwd_d", "bwd_p", "bwd_rows_min", "bwd_pf", "rope_k", "rope_wpb",
 * "rope_groups", "gemm_tile" (1: 128 x 128 outputs per workgroup, 2: 256 x
 * 256), "fwd_pack" (forwards of aligned rows of at most 32 16-byte chunks:
 * 1 one wave per row, 4/8/16/32 that many lanes per row), "bwd_pack" (the
 * same for the backwards).  A key whose forced value
 * does not fit a call's shape makes that call return NR_ERR_SHAPE.
 * Returns NR_ERR_TUNE for an unknown key or a negative value.  Host only.
 */
nr_status_t nr_tune(const char* key, int value);

/*
 * nr_stream_copy -- measurement aid, not part of the method: copies `bytes`
 * bytes from src to dst (device memory, not overlapping) with the access
 * pattern of the row kernels (16-byte streaming loads and stores, one pass,
 * a one-shot grid).  Its bandwidth is the practical HBM ceiling that
 * the norm and RoPE kernels are reported against (the method's benchmark
 * compares fused kernels by the bytes they move).  Both pointers 16-byte
 * aligned and bytes a multiple of 16, else NR_ERR_SHAPE; NR_ERR_ALIAS when
 * the ranges overlap; bytes == 0 is a no-op.  Asynchronous on `stream`.
 */
nr_status_t nr_stream_copy(const void* src, void* dst, size_t bytes, void* stream);

/*
 * nr_stream_mix -- measurement aid like nr_stream_copy, for the other
 * read/write mixes of the path: reads `bytes` bytes from each of a and b
 * and, when write != 0, writes their bitwise xor to dst (two streams read,
 * one written: the backward's mix); when write == 0 nothing is written
 * (dst is only written if the two inputs' xor has an all-ones 16-byte
 * word, so pass inputs whose words are not complements of each other).
 * Same rules as nr_stream_copy (dst may not overlap a or b).
 */
nr_status_t nr_stream_mix(const void* a, const void* b, void* dst, size_t bytes, int write,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NORMROPE_H */
