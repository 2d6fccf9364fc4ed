// norm_bwd_dispatch.hip -- host entry points of the backward (stage 1 by
// dtype, operator and epilogue) and stage 2, the fixed-order column sum.
#include "norm_bwd.hpp"
#include "norm_bwd_long.hpp"

namespace nr {

// Stage 2: out[j] = sum over p of part[p][j].  C columns per workgroup,
// one per lane of each group of C lanes; the 64 / C groups of each of the nw
// waves take the fixed row slices [sP/S, (s+1)P/S), s = wave (64 / C) + group
// of S = nw (64 / C), added in order with 16 loads in flight; the S slice sums
// meet in LDS and are added in slice order.  blockIdx.y selects the matrix
// (dW / dgamma, or dbeta).  The slices, and so the bits of the result, depend
// only on S: 32 columns on 8 waves sum exactly as 64 columns on 16.
template <int C>
__global__ void __launch_bounds__(1024)
colreduce(const float* part, int64_t part_stride, int P, int n, float* out0, float* out1) {
  constexpr int G = 64 / C;
  float* out = blockIdx.y == 0 ? out0 : out1;
  if (out == nullptr) return;  // uniform over the workgroup
  const float* src = part + blockIdx.y * part_stride;
  __shared__ float acc_lds[16 * G][C];
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int ns = (blockDim.x >> 6) * G;
  const int cl = lane % C, sl = wave * G + lane / C;
  const int col = blockIdx.x * C + cl;
  const int p0 = static_cast<int>((static_cast<int64_t>(P) * sl) / ns);
  const int p1 = static_cast<int>((static_cast<int64_t>(P) * (sl + 1)) / ns);
  float s = 0.0f;
  if (col < n) {
    const float* c = src + col;
    int p = p0;
    for (; p + 16 <= p1; p += 16) {
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = c[static_cast<int64_t>(p + i) * n];
#pragma unroll
      for (int i = 0; i < 16; ++i) s += v[i];
    }
    for (; p < p1; ++p) s += c[static_cast<int64_t>(p) * n];
  }
  acc_lds[sl][cl] = s;
  __syncthreads();
  if (sl == 0 && col < n) {
    float tot = acc_lds[0][cl];
    for (int i = 1; i < ns; ++i) tot += acc_lds[i][cl];
    out[col] = tot;
  }
}

#define NR_BWD_EXTERN(T, LN, EPI)                                                             \
  extern template hipError_t launch_bwd_t<T, LN, EPI>(const BwdPlan&, const void*, const void*, \
                                                      const void*, const void*, const float*,    \
                                                      const float*, void*, float*, int64_t, int, \
                                                      float, const RopeArgs&, hipStream_t);
NR_BWD_EXTERN(float, false, kEpiNone)
NR_BWD_EXTERN(bf16, false, kEpiNone)
NR_BWD_EXTERN(float, true, kEpiNone)
NR_BWD_EXTERN(bf16, true, kEpiNone)
NR_BWD_EXTERN(float, false, kEpiRope)
NR_BWD_EXTERN(bf16, false, kEpiRope)
NR_BWD_EXTERN(float, true, kEpiGelu)
NR_BWD_EXTERN(bf16, true, kEpiGelu)
NR_BWD_EXTERN(f16, false, kEpiNone)
NR_BWD_EXTERN(f16, true, kEpiNone)
NR_BWD_EXTERN(f16, false, kEpiRope)
NR_BWD_EXTERN(f16, true, kEpiGelu)
#undef NR_BWD_EXTERN

hipError_t launch_norm_bwd(bool ln, int dt, const BwdPlan& pl, const void* dy, const void* x,
                           const void* w, const float* mean, const float* rstat, void* dx,
                           float* part, int64_t rows, int n, float w_add, hipStream_t st) {
  const RopeArgs none{nullptr, nullptr, 2, 1};
  return by_dtype(dt, [&](auto tag) {
    using T = decltype(tag);
    return ln ? launch_bwd_t<T, true, kEpiNone>(pl, dy, x, w, nullptr, mean, rstat, dx, part, rows, n,
                                                w_add, none, st)
              : launch_bwd_t<T, false, kEpiNone>(pl, dy, x, w, nullptr, mean, rstat, dx, part, rows,
                                                 n, w_add, none, st);
  });
}

hipError_t launch_rms_rope_bwd(int dt, const BwdPlan& pl, const void* dout, const void* x,
                               const void* w, const float* inv_rms, const RopeArgs& ra, void* dx,
                               float* part, int64_t rows, int n, float w_add, hipStream_t st) {
  return by_dtype(dt, [&](auto tag) {
    using T = decltype(tag);
    return launch_bwd_t<T, false, kEpiRope>(pl, dout, x, w, nullptr, nullptr, inv_rms, dx, part,
                                            rows, n, w_add, ra, st);
  });
}

hipError_t launch_ln_gelu_bwd(int dt, const BwdPlan& pl, const void* dout, const void* x,
                              const void* gamma, const void* beta, const float* mean,
                              const float* rstd, void* dx, float* part, int64_t rows, int n,
                              hipStream_t st) {
  const RopeArgs none{nullptr, nullptr, 2, 1};
  return by_dtype(dt, [&](auto tag) {
    using T = decltype(tag);
    return launch_bwd_t<T, true, kEpiGelu>(pl, dout, x, gamma, beta, mean, rstd, dx, part, rows, n,
                                           0.0f, none, st);
  });
}

#define NR_BWD_LONG_EXTERN(T, LN, EPI)                                                         \
  extern template hipError_t launch_bwd_long_t<T, LN, EPI>(                                      \
      bool, const void*, const void*, const void*, const void*, const float*, const float*,     \
      float*, void*, float*, int64_t, int64_t, int, float, const RopeArgs&, hipStream_t);
NR_BWD_LONG_EXTERN(float, false, kEpiNone)
NR_BWD_LONG_EXTERN(bf16, false, kEpiNone)
NR_BWD_LONG_EXTERN(f16, false, kEpiNone)
NR_BWD_LONG_EXTERN(float, true, kEpiNone)
NR_BWD_LONG_EXTERN(bf16, true, kEpiNone)
NR_BWD_LONG_EXTERN(f16, true, kEpiNone)
NR_BWD_LONG_EXTERN(float, false, kEpiRope)
NR_BWD_LONG_EXTERN(bf16, false, kEpiRope)
NR_BWD_LONG_EXTERN(f16, false, kEpiRope)
NR_BWD_LONG_EXTERN(float, true, kEpiGelu)
NR_BWD_LONG_EXTERN(bf16, true, kEpiGelu)
NR_BWD_LONG_EXTERN(f16, true, kEpiGelu)
#undef NR_BWD_LONG_EXTERN

hipError_t launch_norm_bwd_long(int dt, bool ln, int epi, bool aligned, const void* dy,
                                const void* x, const void* w, const void* beta, const float* mean,
                                const float* rstat, float* terms, void* dx, float* part,
                                int64_t P, int64_t rows, int n, float w_add, const RopeArgs& ra,
                                hipStream_t st) {
  return by_dtype(dt, [&](auto tag) {
    using T = decltype(tag);
    if (epi == kEpiRope)
      return launch_bwd_long_t<T, false, kEpiRope>(aligned, dy, x, w, nullptr, nullptr, rstat,
                                                   terms, dx, part, P, rows, n, w_add, ra, st);
    if (epi == kEpiGelu)
      return launch_bwd_long_t<T, true, kEpiGelu>(aligned, dy, x, w, beta, mean, rstat, terms, dx,
                                                  part, P, rows, n, 0.0f, ra, st);
    return ln ? launch_bwd_long_t<T, true, kEpiNone>(aligned, dy, x, w, nullptr, mean, rstat, terms,
                                                     dx, part, P, rows, n, w_add, ra, st)
              : launch_bwd_long_t<T, false, kEpiNone>(aligned, dy, x, w, nullptr, nullptr, rstat,
                                                      terms, dx, part, P, rows, n, w_add, ra, st);
  });
}

hipError_t launch_colreduce(const float* part, int64_t part_stride, int P, int n, float* out0,
                            float* out1, hipStream_t st, int slices) {
  if (slices < 1 || slices > 16) return hipErrorInvalidValue;
  const unsigned ny = out1 != nullptr ? 2u : 1u;
  if (slices == 16) {
    // twice the workgroups of 64 columns on 16 waves, the same sums (the
    // 3840 x 5120 RMSNorm backward: 25.2 -> 24.5 us)
    hipLaunchKernelGGL(colreduce<32>, dim3(static_cast<unsigned>((n + 31) / 32), ny), dim3(512), 0,
                       st, part, part_stride, P, n, out0, out1);
  } else {
    hipLaunchKernelGGL(colreduce<64>, dim3(static_cast<unsigned>((n + 63) / 64), ny),
                       dim3(64 * slices), 0, st, part, part_stride, P, n, out0, out1);
  }
  return hipGetLastError();
}

}  // namespace nr
