// norm_fwd.hpp -- single-pass RMSNorm / LayerNorm forward for gfx950.
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
#pragma once

#include "nr_device.hpp"
#include "nr_internal.hpp"

namespace nr {

// Sum each of the J values over the W waves of a row group (W == 1: pure
// wave reductions).  red: LDS scratch [J][16] used once per call site.
template <int J>
__device__ __forceinline__ void group_sum_n(float (&v)[J], int W, int wave, int g, float (*red)[16]) {
#pragma unroll
  for (int j = 0; j < J; ++j) v[j] = wave_sum(v[j]);
  if (W == 1) return;
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int j = 0; j < J; ++j) red[j][wave] = v[j];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < J; ++j) {
    float s = 0.0f;
    for (int i = 0; i < W; ++i) s += red[j][g * W + i];
    v[j] = s;
  }
}

// Loads the J consecutive rows of a row group starting at row0 (16-byte
// chunks, lane t owning chunks t, t + 64 W, ...).  Rows past the last one see
// an empty buffer: their loads return 0 and move no data.
template <typename T, int K, int J, bool VEC>
__device__ __forceinline__ void fwd_load_rows(u32x4 (&xa)[J * K], const T* x, int64_t row0,
                                              int64_t rows, int n, int t, int nthr) {
  const uint32_t rbytes = static_cast<uint32_t>(n) * sizeof(T);
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t row = row0 + j;
    const bool active = row < rows;
    const rsrc_t xr = make_rsrc(x + (active ? row : 0) * static_cast<int64_t>(n), active ? rbytes : 0u);
#pragma unroll
    for (int k = 0; k < K; ++k) xa[j * K + k] = ld_chunk<T, VEC, kStream>(xr, t + k * nthr);
  }
}

// A row group (W waves) normalises the J consecutive rows it has loaded; the
// weight chunks serve all J of them.  Epilogues, applied before the single
// rounding: kEpiRope (RMSNorm) rotates the normalised row as interleaved RoPE
// pairs by its token's angles, so the norm -> RoPE chain costs one read and
// one write of the row; kEpiGelu (LayerNorm) passes the affine output through
// the tanh-approximated GeLU (LLM层的优化算子, 编写定制融合算子).
// red0, red1: LDS scratch [J][16] for this call's two workgroup reductions;
// a caller that loops hands in a different pair on consecutive calls (the
// reductions have one barrier each, so a pair is free again after the next).
template <typename T, int K, int J, bool VEC, bool LN, int EPI>
__device__ __forceinline__ void fwd_finish_rows(u32x4 (&xa)[J * K], u32x4 (&wa)[K],
                                                u32x4 (&ba)[K], const T* w, T* y, float* stat0,
                                                float* stat1, int64_t row0, int64_t rows, int n,
                                                float eps, float w_add, int W, int wave, int g,
                                                int t, int nthr, const RopeArgs& ra,
                                                float (*red0)[16], float (*red1)[16]) {
  constexpr int E = Vec<T>::N;
  const uint32_t rbytes = static_cast<uint32_t>(n) * sizeof(T);
  const float fn = static_cast<float>(n);
  // without a weight its loads returned 0, and 0 + 1 is the weight 1
  const float wadd = (w != nullptr) ? w_add : 1.0f;
  float mean[J], r[J];
  if constexpr (LN) {
    float s[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      s[j] = 0.0f;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        float v[E];
        unpack<T>(xa[j * K + k], v);
#pragma unroll
        for (int e = 0; e < E; ++e) s[j] += v[e];
      }
    }
    group_sum_n<J>(s, W, wave, g, red0);
    reload_barrier<J * K>(xa);
    // second pass over the registers, not over HBM: squared deviations.
    // The slots past n (read as 0) are left out; when the row fills every
    // slot of the row group exactly (5120 bf16 on 2 waves of 5 chunks) no
    // slot is masked, a uniform branch.
    float q[J];
    const bool full = nthr * K * E == n;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      mean[j] = s[j] / fn;
      q[j] = 0.0f;
      if (full) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
          float v[E];
          unpack<T>(xa[j * K + k], v);
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float d = v[e] - mean[j];
            q[j] = fmaf(d, d, q[j]);
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const int c = t + k * nthr;
          float v[E];
          unpack<T>(xa[j * K + k], v);
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float d = (c * E + e < n) ? v[e] - mean[j] : 0.0f;
            q[j] = fmaf(d, d, q[j]);
          }
        }
      }
    }
    group_sum_n<J>(q, W, wave, g, red1);
#pragma unroll
    for (int j = 0; j < J; ++j) r[j] = rsqrtf(q[j] / fn + eps);
  } else {
    float ss[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      ss[j] = 0.0f;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        float v[E];
        unpack<T>(xa[j * K + k], v);
#pragma unroll
        for (int e = 0; e < E; ++e) ss[j] = fmaf(v[e], v[e], ss[j]);
      }
    }
    group_sum_n<J>(ss, W, wave, g, red0);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      mean[j] = 0.0f;
      r[j] = rsqrtf(ss[j] / fn + eps);
    }
  }
  reload_barrier<J * K>(xa);
  // the weights too: widen them where they are used, not when they arrive
  reload_barrier<K>(wa);
  if constexpr (LN) reload_barrier<K>(ba);

#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t row = row0 + j;
    const bool active = row < rows;
    const rsrc_t yr = make_rsrc(y + (active ? row : 0) * static_cast<int64_t>(n), active ? rbytes : 0u);
    // RoPE: the token's table rows, and the offset within its head of this
    // lane's first chunk (advancing by a fixed step per chunk)
    const int half = ra.head_dim >> 1;
    constexpr bool ROPE = EPI == kEpiRope;
    const int64_t tok = ROPE ? (active ? row : 0) / ra.rows_per_token : 0;
    const uint32_t tb = (ROPE && active) ? static_cast<uint32_t>(half) * 4u : 0u;
    const rsrc_t cr = make_rsrc(ra.cos_tab + tok * half, tb);
    const rsrc_t sr = make_rsrc(ra.sin_tab + tok * half, tb);
    int hoff = ROPE ? (t * E) % ra.head_dim : 0;
    const int hstep = ROPE ? (nthr * E) % ra.head_dim : 0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      float v[E], wv[E], bv[E], o[E];
      unpack<T>(xa[j * K + k], v);
      unpack<T>(wa[k], wv);
      if constexpr (LN) unpack<T>(ba[k], bv);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float ww = wv[e] + wadd;
        if constexpr (LN) {
          o[e] = fmaf((v[e] - mean[j]) * r[j], ww, bv[e]);
          if constexpr (EPI == kEpiGelu) o[e] = gelu_tanh(o[e]);
        } else {
          o[e] = (v[e] * r[j]) * ww;
        }
      }
      if constexpr (ROPE) {
        constexpr int PP = E / 2;
        float cf[PP], sf[PP];
        if constexpr (VEC) {
          // whole chunks lie inside one head: PP consecutive pairs
          load_tab<PP>(cr, hoff >> 1, cf);
          load_tab<PP>(sr, hoff >> 1, sf);
        } else {
#pragma unroll
          for (int p = 0; p < PP; ++p) {
            const int ho = (hoff + 2 * p) % ra.head_dim;
            cf[p] = ld_f32(cr, (ho >> 1) * 4);
            sf[p] = ld_f32(sr, (ho >> 1) * 4);
          }
        }
        rotate_pairs<PP>(o, cf, sf, 1.0f);
        hoff += hstep;
        if (hoff >= ra.head_dim) hoff -= ra.head_dim;
      }
      st_chunk<T, VEC, kNormStore>(yr, t + k * nthr, pack<T>(o));
    }
    if (active && t == 0) {
      if constexpr (LN) {
        if (stat0) stat0[row] = mean[j];
        if (stat1) stat1[row] = r[j];
      } else {
        if (stat0) stat0[row] = r[j];
      }
    }
  }
}

template <typename T, int K, bool VEC, bool LN>
__device__ __forceinline__ void fwd_load_weights(u32x4 (&wa)[K], u32x4 (&ba)[K], const T* w,
                                                 const T* b, int n, int t, int nthr) {
  const uint32_t rbytes = static_cast<uint32_t>(n) * sizeof(T);
  const rsrc_t wr = make_rsrc(w, w != nullptr ? rbytes : 0u);
  const rsrc_t br = make_rsrc(b, b != nullptr ? rbytes : 0u);
#pragma unroll
  for (int k = 0; k < K; ++k) {
    wa[k] = ld_chunk<T, VEC>(wr, t + k * nthr);
    if constexpr (LN) ba[k] = ld_chunk<T, VEC>(br, t + k * nthr);
  }
}

// One-shot form: each row group of the grid normalises its J rows once.
template <typename T, int K, int J, bool VEC, bool LN, int EPI>
__device__ __forceinline__ void norm_fwd_body(const T* x, const T* w, const T* b, T* y,
                                              float* stat0, float* stat1, int64_t rows, int n,
                                              float eps, float w_add, int W, const RopeArgs& ra) {
  __shared__ float red0[J][16], red1[J][16];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int g = wave / W;
  const int t = (wave - g * W) * 64 + lane;
  const int nthr = 64 * W;
  const int R = blockDim.x / nthr;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * R + g) * J;
  u32x4 xa[J * K], wa[K], ba[K];
  fwd_load_rows<T, K, J, VEC>(xa, x, row0, rows, n, t, nthr);
  fwd_load_weights<T, K, VEC, LN>(wa, ba, w, b, n, t, nthr);
  fwd_finish_rows<T, K, J, VEC, LN, EPI>(xa, wa, ba, w, y, stat0, stat1, row0, rows, n, eps, w_add,
                                         W, wave, g, t, nthr, ra, red0, red1);
}

// One wavefront per row group (W == 1), at most 4 row groups (256 threads)
// per workgroup.
template <typename T, int K, int J, bool VEC, bool LN, int EPI>
__global__ void __launch_bounds__(256)
norm_fwd_wave(const T* x, const T* w, const T* b, T* y, float* stat0, float* stat1,
              int64_t rows, int n, float eps, float w_add, RopeArgs ra) {
  norm_fwd_body<T, K, J, VEC, LN, EPI>(x, w, b, y, stat0, stat1, rows, n, eps, w_add, 1, ra);
}

// Several waves per row group (W > 1), up to 16 waves per workgroup.
template <typename T, int K, int J, bool VEC, bool LN, int EPI>
__global__ void __launch_bounds__(1024)
norm_fwd_group(const T* x, const T* w, const T* b, T* y, float* stat0, float* stat1,
               int64_t rows, int n, float eps, float w_add, int W, RopeArgs ra) {
  norm_fwd_body<T, K, J, VEC, LN, EPI>(x, w, b, y, stat0, stat1, rows, n, eps, w_add, W, ra);
}


template <typename T, int K, int J, bool A, bool LN, int RP>
hipError_t launch_fwd_kj(const FwdPlan& pl, const void* x, const void* w, const void* b, void* y,
                         float* s0, float* s1, int64_t rows, int n, float eps, float w_add,
                         const RopeArgs& ra, hipStream_t st) {
  const int64_t per_block = static_cast<int64_t>(pl.R) * J;
  const int64_t blocks = (rows + per_block - 1) / per_block;
  const dim3 block(64 * pl.W * pl.R);
  const dim3 grid(static_cast<unsigned>(blocks));
  if (pl.W == 1) {
    hipLaunchKernelGGL((norm_fwd_wave<T, K, J, A, LN, RP>), grid, block, 0, st,
                       static_cast<const T*>(x), static_cast<const T*>(w),
                       static_cast<const T*>(b), static_cast<T*>(y), s0, s1, rows, n, eps, w_add,
                       ra);
  } else if constexpr (K * J <= 10 && K <= 8) {
    hipLaunchKernelGGL((norm_fwd_group<T, K, J, A, LN, RP>), grid, block, 0, st,
                       static_cast<const T*>(x), static_cast<const T*>(w),
                       static_cast<const T*>(b), static_cast<T*>(y), s0, s1, rows, n, eps, w_add,
                       pl.W, ra);
  } else {
    return hipErrorInvalidValue;  // the planner keeps K <= 8 and K * J <= 10 when W > 1
  }
  return hipGetLastError();
}

template <typename T, int K, bool A, bool LN, int RP>
hipError_t launch_fwd_k(const FwdPlan& pl, const void* x, const void* w, const void* b, void* y,
                        float* s0, float* s1, int64_t rows, int n, float eps, float w_add,
                        const RopeArgs& ra, hipStream_t st) {
  if constexpr (K <= 5) {
    if (pl.J == 2)
      return launch_fwd_kj<T, K, 2, A, LN, RP>(pl, x, w, b, y, s0, s1, rows, n, eps, w_add, ra, st);
  }
  if (pl.J != 1) return hipErrorInvalidValue;
  return launch_fwd_kj<T, K, 1, A, LN, RP>(pl, x, w, b, y, s0, s1, rows, n, eps, w_add, ra, st);
}

template <typename T, bool A, bool LN, int RP>
hipError_t launch_fwd_a(const FwdPlan& pl, const void* x, const void* w, const void* b, void* y,
                        float* s0, float* s1, int64_t rows, int n, float eps, float w_add,
                        const RopeArgs& ra, hipStream_t st) {
  switch (pl.K) {
#define NR_CASE(KK) \
  case KK: return launch_fwd_k<T, KK, A, LN, RP>(pl, x, w, b, y, s0, s1, rows, n, eps, w_add, ra, st);
    NR_CASE(1) NR_CASE(2) NR_CASE(4) NR_CASE(5) NR_CASE(6) NR_CASE(8) NR_CASE(10)
#undef NR_CASE
    default: return hipErrorInvalidValue;
  }
}

template <typename T, bool LN, int RP>
hipError_t launch_fwd_t(const FwdPlan& pl, const void* x, const void* w, const void* b, void* y,
                        float* s0, float* s1, int64_t rows, int n, float eps, float w_add,
                        const RopeArgs& ra, hipStream_t st) {
  return pl.aligned ? launch_fwd_a<T, true, LN, RP>(pl, x, w, b, y, s0, s1, rows, n, eps, w_add, ra, st)
                    : launch_fwd_a<T, false, LN, RP>(pl, x, w, b, y, s0, s1, rows, n, eps, w_add, ra, st);
}


// One translation unit instantiates each (type, operator, epilogue)
// combination, so the build compiles them in parallel.
#define NR_FWD_INSTANTIATE(T, LN, EPI)                                                         \
  template hipError_t launch_fwd_t<T, LN, EPI>(const FwdPlan&, const void*, const void*,       \
                                               const void*, void*, float*, float*, int64_t, int, \
                                               float, float, const RopeArgs&, hipStream_t);

}  // namespace nr
