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
  int S = 0;  // > 0: rows of at most S chunks, S lanes each (norm_fwd_packed)
};

// Backward stage 1: P workgroups of W waves, D rows per batch, K chunks per
// lane, PF batches loaded ahead.
struct BwdPlan {
  int W, K, D, P, PF;
  int64_t rows_per_block;
  bool aligned;
  bool lacc;  // dW accumulators in LDS (plain RMSNorm, 32 elements a lane)
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
// (norm_bwd_long.hpp).  Its pass B runs P row groups times S column slices
// of kLongSliceChunks 16-byte chunks, with P = min(ceil(rows / 16),
// max(1, 256 / S)): about one workgroup per CU.  Fewer, longer row streams
// measured fastest (bf16 LayerNorm backward of 4096 rows of 65536: 447 us
// at 256 workgroups, 460 at 512, 499 at 2048); past one per CU the extra
// streams only add open DRAM pages.  P is a function of the shape and the
// element size alone, so the summation order does not depend on the device.
constexpr int64_t kLongRowMin = 16385;
constexpr int kLongSliceChunks = 512;
// The plain RMSNorm backward of 16-byte-aligned 16-bit rows keeps one pass
// up to 32768 elements, its dW accumulators in LDS (norm_bwd.hpp; for fp32
// or element-wise rows the same kernel spilled).  Every other backward takes
// two passes from kLongRowMin on.
constexpr int64_t kRmsOnePassMax = 32768;
inline bool bwd_two_pass(bool rms_one_pass_ok, int64_t n) {
  return n >= kLongRowMin && (!rms_one_pass_ok || n > kRmsOnePassMax);
}
inline int64_t long_bwd_groups(int64_t rows, int64_t n, int elem_bytes) {
  const int64_t chunks = (n * elem_bytes + 15) / 16;
  const int64_t slices = (chunks + kLongSliceChunks - 1) / kLongSliceChunks;
  int64_t cap = 256 / slices;
  if (cap < 1) cap = 1;
  int64_t p = (rows + 15) / 16;
  if (p > cap) p = cap;
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
// LayerNorm + GeLU backward, stage 1, on 16-bit rows of 640 W elements (W =
// 4 or 8) with 10 elements a lane: W waves, the same number on every SIMD.
bool ln_gelu_pair_fits(int dt, int64_t n, bool aligned);
hipError_t launch_ln_gelu_bwd_pair(int dt, int P, const void* dout, const void* x,
                                   const void* gamma, const void* beta, const float* mean,
                                   const float* rstd, void* dx, float* part, int64_t rows, int n,
                                   hipStream_t st);
// Rows of at most pl.S whole chunks, 64 / pl.S of them side by side in a
// wave (pl.S = 4, 8, 16 or 32; aligned rows only); epi as the row kernels.
int fwd_packed_rows_per_block(int S);
hipError_t launch_fwd_packed(int dt, bool ln, int epi, const FwdPlan& pl, const void* x,
                             const void* w, const void* b, void* y, float* s0, float* s1,
                             int64_t rows, int n, float eps, float w_add, const RopeArgs& ra,
                             hipStream_t st);
// Backward stage 1 of rows of at most S whole chunks (S = 4, 8, 16 or 32),
// 64 / S rows side by side in a wave; P workgroups of four waves take the
// batches of bwd_packed_rows_per_wave(S) rows round-robin.
int bwd_packed_rows_per_wave(int S);
// epi: kEpiNone, kEpiRope (RMSNorm) or kEpiGelu (LayerNorm; b = beta).
hipError_t launch_bwd_packed(int dt, bool ln, int epi, int S, int P, const void* dy,
                             const void* x, const void* w, const void* b, const float* mean,
                             const float* rstat, void* dx, float* part, int64_t rows, int n,
                             float w_add, const RopeArgs& ra, hipStream_t st);
hipError_t launch_norm_fwd(bool ln, int dt, const FwdPlan& pl, const void* x, const void* w,
                           const void* b, void* y, float* s0, float* s1, int64_t rows, int n,
                           float eps, float w_add, hipStream_t st);
hipError_t launch_norm_bwd(bool ln, int dt, const BwdPlan& pl, const void* dy, const void* x,
                           const void* w, const float* mean, const float* rstat, void* dx,
                           float* part, int64_t rows, int n, float w_add, hipStream_t st);
// slices: 1..16 row slices of the P partial rows, summed in order (16 for
// the short-row backward; the long-row one, with few partial rows and
// n/64 >= 256 column workgroups, takes about P/4)
hipError_t launch_colreduce(const float* part, int64_t part_stride, int P, int n, float* out0,
                            float* out1, hipStream_t st, int slices = 16);
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
// LayerNorm -> linear on the 256 x 256 tile (N % 256 == 0); workspace:
// layernorm_linear_ws_bytes(M, N, K, gamma != nullptr) bytes: mean, rstd
// (used when the caller's pointers are null), c_n, d_n, each padded to 256
// bytes, then the folded weight (N K bf16) when gamma is given
inline size_t layernorm_linear_ws_bytes(int64_t M, int64_t N, int64_t K, bool has_gamma) {
  return 2 * linear_rows_bytes(M) + 2 * linear_rows_bytes(N) +
         (has_gamma ? static_cast<size_t>(N * K) * 2 : 0);
}
hipError_t launch_layernorm_linear(const void* x, const void* gamma, const void* beta,
                                   const void* W, void* out, float* mean, float* rstd, void* ws,
                                   int M, int N, int K, float eps, hipStream_t st);
// Wf[n][k] = bf16(W[n][k] (wn[k] + w_add)); N K % 8 == 0, 16-byte aligned
hipError_t launch_fold_norm_weight(const void* wn, const void* W, void* Wf, int64_t N, int K,
                                   float w_add, hipStream_t st);
// Keeps e as the calling thread's last HIP error (nr_last_hip_error) and
// returns the NR_ERR_HIP status code.
int record_hip_error(hipError_t e);
hipError_t launch_stream_copy(const void* src, void* dst, int64_t nvec, hipStream_t st);
hipError_t launch_stream_mix(const void* a, const void* b, void* dst, int64_t nvec, bool write,
                             hipStream_t st);
hipError_t launch_rope_table_3d(float* cos_tab, float* sin_tab, int64_t frames, int64_t height,
                                int64_t width, int pt, int ph, int pw, double theta,
                                hipStream_t st);

}  // namespace nr
