// norm_fwd_dispatch.hip -- host entry points of the forward row kernels,
// choosing the instantiation by dtype, operator and epilogue.
#include "norm_fwd.hpp"

namespace nr {

#define NR_FWD_EXTERN(T, LN, EPI)                                                             \
  extern template hipError_t launch_fwd_t<T, LN, EPI>(const FwdPlan&, const void*, const void*, \
                                                      const void*, void*, float*, float*, int64_t, \
                                                      int, float, float, const RopeArgs&,       \
                                                      hipStream_t);
NR_FWD_EXTERN(float, false, kEpiNone)
NR_FWD_EXTERN(bf16, false, kEpiNone)
NR_FWD_EXTERN(float, true, kEpiNone)
NR_FWD_EXTERN(bf16, true, kEpiNone)
NR_FWD_EXTERN(float, false, kEpiRope)
NR_FWD_EXTERN(bf16, false, kEpiRope)
NR_FWD_EXTERN(float, true, kEpiGelu)
NR_FWD_EXTERN(bf16, true, kEpiGelu)
NR_FWD_EXTERN(f16, false, kEpiNone)
NR_FWD_EXTERN(f16, true, kEpiNone)
NR_FWD_EXTERN(f16, false, kEpiRope)
NR_FWD_EXTERN(f16, true, kEpiGelu)
#undef NR_FWD_EXTERN

hipError_t launch_norm_fwd(bool ln, int dt, const FwdPlan& pl, const void* x, const void* w,
                           const void* b, void* y, float* s0, float* s1, int64_t rows, int n,
                           float eps, float w_add, hipStream_t st) {
  const RopeArgs none{nullptr, nullptr, 2, 1};
  if (pl.S > 0)
    return launch_fwd_packed(dt, ln, kEpiNone, pl, x, w, b, y, s0, s1, rows, n, eps, w_add, none, st);
  return by_dtype(dt, [&](auto tag) {
    using T = decltype(tag);
    return ln ? launch_fwd_t<T, true, kEpiNone>(pl, x, w, b, y, s0, s1, rows, n, eps, w_add, none, st)
              : launch_fwd_t<T, false, kEpiNone>(pl, x, w, b, y, s0, s1, rows, n, eps, w_add, none, st);
  });
}

hipError_t launch_rms_rope_fwd(int dt, const FwdPlan& pl, const void* x, const void* w, void* y,
                               float* inv_rms, const RopeArgs& ra, int64_t rows, int n, float eps,
                               float w_add, hipStream_t st) {
  if (pl.S > 0)
    return launch_fwd_packed(dt, false, kEpiRope, pl, x, w, nullptr, y, inv_rms, nullptr, rows, n,
                             eps, w_add, ra, st);
  return by_dtype(dt, [&](auto tag) {
    using T = decltype(tag);
    return launch_fwd_t<T, false, kEpiRope>(pl, x, w, nullptr, y, inv_rms, nullptr, rows, n, eps,
                                            w_add, ra, st);
  });
}

hipError_t launch_ln_gelu_fwd(int dt, const FwdPlan& pl, const void* x, const void* gamma,
                              const void* beta, void* y, float* mean, float* rstd, int64_t rows,
                              int n, float eps, hipStream_t st) {
  const RopeArgs none{nullptr, nullptr, 2, 1};
  if (pl.S > 0)
    return launch_fwd_packed(dt, true, kEpiGelu, pl, x, gamma, beta, y, mean, rstd, rows, n, eps,
                             0.0f, none, st);
  return by_dtype(dt, [&](auto tag) {
    using T = decltype(tag);
    return launch_fwd_t<T, true, kEpiGelu>(pl, x, gamma, beta, y, mean, rstd, rows, n, eps, 0.0f,
                                           none, st);
  });
}

}  // namespace nr
