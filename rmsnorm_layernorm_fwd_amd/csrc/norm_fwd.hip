// norm_fwd.hip -- single-pass RMSNorm / LayerNorm forward for gfx950.
//
// Operation (Helios 性能优化全解析, 内核一 FlashNorm): each row is read from
// HBM once; its sums are formed on chip; the normalised row, scaled by the
// weight (or by 1 + w for the Gemma variant), is written once; the per-row
// inverse root (and, for LayerNorm, the mean) is stored for the backward.
// All arithmetic is fp32 whatever the storage type and every output is
// rounded once (Janus-Pro-7B模型推理加速实战, 3. 计算精度优化: norms run in
// FP32 and the result is cast back).
//
// Mapping: a row group of W waves owns one row.  W = 1 -- one wavefront per
// row, four rows per workgroup -- whenever the row fits in 64 lanes x K
// chunks (up to 640 chunks: 5120 bf16 or 2560 fp32); that case needs no LDS
// and no barrier, the row sum being a DPP / permlane wave reduction.  Longer
// rows use W > 1 waves whose wave sums meet in LDS.  All of a lane's loads
// (row chunks and weight chunks) are issued before the first use, so each
// wave keeps up to K x 1 KiB of row data in flight.
#include "nr_device.hpp"
#include "nr_internal.hpp"

namespace nr {

template <typename T, int K, bool VEC, bool LN>
__device__ __forceinline__ void norm_fwd_body(const T* x, const T* w, const T* b, T* y,
                                              float* stat0, float* stat1, int64_t rows, int n,
                                              float eps, float w_add, int W) {
  constexpr int E = Vec<T>::N;
  __shared__ float red0[16], red1[16];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int g = wave / W;
  const int t = (wave - g * W) * 64 + lane;
  const int nthr = 64 * W;
  const int R = blockDim.x / nthr;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * R + g;
  const bool active = row < rows;
  const uint32_t rbytes = static_cast<uint32_t>(n) * sizeof(T);
  // a row group past the last row sees an empty buffer: loads give 0, stores vanish
  const rsrc_t xr = make_rsrc(x + (active ? row : 0) * static_cast<int64_t>(n), active ? rbytes : 0u);
  const rsrc_t yr = make_rsrc(y + (active ? row : 0) * static_cast<int64_t>(n), active ? rbytes : 0u);
  const rsrc_t wr = make_rsrc(w, w != nullptr ? rbytes : 0u);
  const rsrc_t br = make_rsrc(b, b != nullptr ? rbytes : 0u);

  u32x4 xa[K], wa[K], ba[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int c = t + k * nthr;
    xa[k] = ld_chunk<T, VEC, kStream>(xr, c);
    wa[k] = ld_chunk<T, VEC>(wr, c);
    if constexpr (LN) ba[k] = ld_chunk<T, VEC>(br, c);
  }

  const float fn = static_cast<float>(n);
  float mean = 0.0f, r;
  if constexpr (LN) {
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      float v[E];
      unpack<T>(xa[k], v);
#pragma unroll
      for (int e = 0; e < E; ++e) s += v[e];
    }
    mean = group_sum(s, W, wave, g, red0) / fn;
    // second pass over the registers, not over HBM: squared deviations
    float q = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int c = t + k * nthr;
      float v[E];
      unpack<T>(xa[k], v);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float d = (c * E + e < n) ? v[e] - mean : 0.0f;
        q = fmaf(d, d, q);
      }
    }
    r = rsqrtf(group_sum(q, W, wave, g, red1) / fn + eps);
  } else {
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      float v[E];
      unpack<T>(xa[k], v);
#pragma unroll
      for (int e = 0; e < E; ++e) ss = fmaf(v[e], v[e], ss);
    }
    r = rsqrtf(group_sum(ss, W, wave, g, red0) / fn + eps);
  }
  reload_barrier<K>(xa);

#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int c = t + k * nthr;
    float v[E], wv[E], bv[E], o[E];
    unpack<T>(xa[k], v);
    unpack<T>(wa[k], wv);
    if constexpr (LN) unpack<T>(ba[k], bv);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float ww = (w != nullptr) ? wv[e] + w_add : 1.0f;
      if constexpr (LN) {
        o[e] = fmaf((v[e] - mean) * r, ww, bv[e]);
      } else {
        o[e] = (v[e] * r) * ww;
      }
    }
    st_chunk<T, VEC, kStream>(yr, c, pack<T>(o));
  }
  if (active && t == 0) {
    if constexpr (LN) {
      if (stat0) stat0[row] = mean;
      if (stat1) stat1[row] = r;
    } else {
      if (stat0) stat0[row] = r;
    }
  }
}

// One wavefront per row (W == 1), at most 4 rows (256 threads) per workgroup,
// so the compiler may spend up to 128 VGPRs per lane keeping a row resident.
template <typename T, int K, bool VEC, bool LN>
__global__ void __launch_bounds__(256)
norm_fwd_wave(const T* x, const T* w, const T* b, T* y, float* stat0, float* stat1,
              int64_t rows, int n, float eps, float w_add) {
  norm_fwd_body<T, K, VEC, LN>(x, w, b, y, stat0, stat1, rows, n, eps, w_add, 1);
}

// Several waves per row (W > 1), up to 16 waves per workgroup.
template <typename T, int K, bool VEC, bool LN>
__global__ void __launch_bounds__(1024)
norm_fwd_group(const T* x, const T* w, const T* b, T* y, float* stat0, float* stat1,
               int64_t rows, int n, float eps, float w_add, int W) {
  norm_fwd_body<T, K, VEC, LN>(x, w, b, y, stat0, stat1, rows, n, eps, w_add, W);
}

namespace {

template <typename T, int K, bool A, bool LN>
hipError_t launch_fwd_k(const FwdPlan& pl, const void* x, const void* w, const void* b, void* y,
                        float* s0, float* s1, int64_t rows, int n, float eps, float w_add,
                        hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((rows + pl.R - 1) / pl.R));
  const dim3 block(64 * pl.W * pl.R);
  if (pl.W == 1) {
    hipLaunchKernelGGL((norm_fwd_wave<T, K, A, LN>), grid, block, 0, st,
                       static_cast<const T*>(x), static_cast<const T*>(w),
                       static_cast<const T*>(b), static_cast<T*>(y), s0, s1, rows, n, eps, w_add);
  } else if constexpr (K <= 8) {
    hipLaunchKernelGGL((norm_fwd_group<T, K, A, LN>), grid, block, 0, st,
                       static_cast<const T*>(x), static_cast<const T*>(w),
                       static_cast<const T*>(b), static_cast<T*>(y), s0, s1, rows, n, eps, w_add,
                       pl.W);
  } else {
    return hipErrorInvalidValue;  // the planner never pairs W > 1 with K > 8
  }
  return hipGetLastError();
}

template <typename T, bool A, bool LN>
hipError_t launch_fwd_a(const FwdPlan& pl, const void* x, const void* w, const void* b, void* y,
                        float* s0, float* s1, int64_t rows, int n, float eps, float w_add,
                        hipStream_t st) {
  switch (pl.K) {
#define NR_CASE(KK) \
  case KK: return launch_fwd_k<T, KK, A, LN>(pl, x, w, b, y, s0, s1, rows, n, eps, w_add, st);
    NR_CASE(1) NR_CASE(2) NR_CASE(4) NR_CASE(5) NR_CASE(6) NR_CASE(8) NR_CASE(10)
#undef NR_CASE
    default: return hipErrorInvalidValue;
  }
}

template <typename T, bool LN>
hipError_t launch_fwd_t(const FwdPlan& pl, const void* x, const void* w, const void* b, void* y,
                        float* s0, float* s1, int64_t rows, int n, float eps, float w_add,
                        hipStream_t st) {
  return pl.aligned ? launch_fwd_a<T, true, LN>(pl, x, w, b, y, s0, s1, rows, n, eps, w_add, st)
                    : launch_fwd_a<T, false, LN>(pl, x, w, b, y, s0, s1, rows, n, eps, w_add, st);
}

}  // namespace

hipError_t launch_norm_fwd(bool ln, int dt, const FwdPlan& pl, const void* x, const void* w,
                           const void* b, void* y, float* s0, float* s1, int64_t rows, int n,
                           float eps, float w_add, hipStream_t st) {
  if (dt == kF32)
    return ln ? launch_fwd_t<float, true>(pl, x, w, b, y, s0, s1, rows, n, eps, w_add, st)
              : launch_fwd_t<float, false>(pl, x, w, b, y, s0, s1, rows, n, eps, w_add, st);
  return ln ? launch_fwd_t<bf16, true>(pl, x, w, b, y, s0, s1, rows, n, eps, w_add, st)
            : launch_fwd_t<bf16, false>(pl, x, w, b, y, s0, s1, rows, n, eps, w_add, st);
}

}  // namespace nr
