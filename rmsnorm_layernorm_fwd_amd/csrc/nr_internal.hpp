// nr_internal.hpp -- launch plans and launcher entry points shared between
// the kernel translation units and the C-ABI layer (api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nr {

constexpr int kF32 = 0;   // matches NR_F32
constexpr int kBF16 = 1;  // matches NR_BF16
constexpr int kF16 = 2;   // matches NR_F16

// Forward row kernel: W waves per row group, K 16-byte chunks per lane, J
// rows per row group, R row groups per workgroup.  aligned: 128-bit
// loads/stores on every row.
struct FwdPlan {
  int W, K, R, J;
  bool aligned;
};

// Backward stage 1: P workgroups of W waves, D rows per batch, K chunks per
// lane, PF batches loaded ahead.
struct BwdPlan {
  int W, K, D, P, PF;
  int64_t rows_per_block;
  bool aligned;
};

// RoPE: `groups` waves per token, each taking K chunks per lane per pass
// over the heads; waves_per_block waves per workgroup.  aligned: 128-bit
// path; fast: the table slice a lane needs is the same for every chunk it
// owns.
struct RopePlan {
  int K, waves_per_block, groups;
  bool aligned, fast;
};

// Interleaved-RoPE epilogue of the fused RMSNorm + RoPE kernels: row i
// belongs to token i / rows_per_token, whose table row has head_dim / 2
// entries; the row is n / head_dim consecutive head vectors.
struct RopeArgs {
  const float* cos_tab;
  const float* sin_tab;
  int head_dim;
  int64_t rows_per_token;
};

// Rows of at least kLongRowMin elements take the two-pass backward
// (norm_bwd_long.hpp).  Its pass B uses long_bwd_groups(rows) row groups:
// a function of the row count only, so the summation order and the
// workspace size do not depend on the device.
constexpr int64_t kLongRowMin = 16385;
inline int64_t long_bwd_groups(int64_t rows) {
  int64_t p = (rows + 15) / 16;
  if (p > 128) p = 128;
  return p < 1 ? 1 : p;
}

// epi: 0 none, 1 RoPE (RMSNorm only), 2 GeLU (LayerNorm only).  terms:
// fp32 [rows][2] scratch; part: fp32 [2][P][n] partial rows or null.
hipError_t launch_norm_bwd_long(int dt, bool ln, int epi, bool aligned, const void* dy,
                                const void* x, const void* w, const void* beta, const float* mean,
                                const float* rstat, float* terms, void* dx, float* part,
                                int64_t P, int64_t rows, int n, float w_add, const RopeArgs& ra,
                                hipStream_t st);
hipError_t launch_rms_rope_fwd(int dt, const FwdPlan& pl, const void* x, const void* w, void* y,
                               float* inv_rms, const RopeArgs& ra, int64_t rows, int n, float eps,
                               float w_add, hipStream_t st);
hipError_t launch_rms_rope_bwd(int dt, const BwdPlan& pl, const void* dout, const void* x,
                               const void* w, const float* inv_rms, const RopeArgs& ra, void* dx,
                               float* part, int64_t rows, int n, float w_add, hipStream_t st);
hipError_t launch_ln_gelu_fwd(int dt, const FwdPlan& pl, const void* x, const void* gamma,
                              const void* beta, void* y, float* mean, float* rstd, int64_t rows,
                              int n, float eps, hipStream_t st);
hipError_t launch_ln_gelu_bwd(int dt, const BwdPlan& pl, const void* dout, const void* x,
                              const void* gamma, const void* beta, const float* mean,
                              const float* rstd, void* dx, float* part, int64_t rows, int n,
                              hipStream_t st);
hipError_t launch_norm_fwd(bool ln, int dt, const FwdPlan& pl, const void* x, const void* w,
                           const void* b, void* y, float* s0, float* s1, int64_t rows, int n,
                           float eps, float w_add, hipStream_t st);
hipError_t launch_norm_bwd(bool ln, int dt, const BwdPlan& pl, const void* dy, const void* x,
                           const void* w, const float* mean, const float* rstat, void* dx,
                           float* part, int64_t rows, int n, float w_add, hipStream_t st);
hipError_t launch_colreduce(const float* part, int64_t part_stride, int P, int n, float* out0,
                            float* out1, hipStream_t st);
hipError_t launch_rope(int dt, const RopePlan& pl, void* x, const float* cos_tab,
                       const float* sin_tab, int64_t batch, int64_t tokens, int heads,
                       int head_dim, int64_t sb, int64_t st_, int64_t sh, float sign,
                       hipStream_t st);
hipError_t launch_rope_table_1d(float* cos_tab, float* sin_tab, int64_t tokens, int head_dim,
                                int64_t pos0, double theta, hipStream_t st);
// tile: 1 = 128 x 128 outputs per workgroup (W scaled by the norm weight in
// the kernel, no workspace), 2 = 256 x 256 (N % 256 == 0): the row
// statistics first (into inv_rms, else the workspace's first
// linear_rows_bytes(M) bytes), then with a norm weight W folded into the
// workspace after them (N K bf16)
inline size_t linear_rows_bytes(int64_t M) { return static_cast<size_t>((M * 4 + 255) / 256 * 256); }
hipError_t launch_rmsnorm_linear(const void* x, const void* wn, const void* W, void* out,
                                 float* inv_rms, void* ws, int M, int N, int K, float eps,
                                 float w_add, int tile, hipStream_t st);
// Wf[n][k] = bf16(W[n][k] (wn[k] + w_add)); N K % 8 == 0, 16-byte aligned
hipError_t launch_fold_norm_weight(const void* wn, const void* W, void* Wf, int64_t N, int K,
                                   float w_add, hipStream_t st);
hipError_t launch_stream_copy(const void* src, void* dst, int64_t nvec, hipStream_t st);
hipError_t launch_rope_table_3d(float* cos_tab, float* sin_tab, int64_t frames, int64_t height,
                                int64_t width, int pt, int ph, int pw, double theta,
                                hipStream_t st);

}  // namespace nr
