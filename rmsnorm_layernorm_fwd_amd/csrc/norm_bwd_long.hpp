// norm_bwd_long.hpp -- the norm backward for rows longer than 16384
// elements.
//
// The single-pass backward (norm_bwd.hpp) keeps, in every lane, the fp32
// column accumulators and weights of the columns it owns, for a whole row
// spread over one workgroup.  Past 16384 elements a row's column state no
// longer fits a workgroup's registers (a 65536-wide LayerNorm row needs
// 512 KiB of fp32 accumulators: a CU's whole register file), the kernel
// spills and falls to a fraction of the memory bandwidth.  Long rows take
// two passes instead:
//
//   A  one workgroup per row reads x and dy and stores the row's two
//      reduction terms (RMSNorm: mean(g xhat); LayerNorm: mean(g) and
//      mean(g xhat), g = dy w') into an fp32 [rows][2] scratch array;
//   B  the columns are split into slices of 512 16-byte chunks; workgroup
//      (p, s) takes slice s of rows p, p + P, p + 2P, ..., computes dx from
//      the row terms of pass A with no reduction at all, and accumulates the
//      slice's column partials in registers, written once as partial row p.
//
// Stage 2 (colreduce) then adds the P partial rows in order, as for short
// rows.  Pass A re-reads x and dy, so long rows move 10n instead of 6n bytes
// per 16-bit row; every summation order is still fixed by the shape.
#pragma once

#include "norm_bwd.hpp"

namespace nr {

constexpr int kSplitLanes = 256;  // pass B: 4 waves per workgroup
constexpr int kSplitK = 2;        // pass B: chunks per lane (slice = 512 chunks)
static_assert(kSplitLanes * kSplitK == kLongSliceChunks, "the host sizes P by this slice width");

// cos / sin of the pairs in chunk c of a row whose table row is at cr / sr
template <typename T, bool VEC>
__device__ __forceinline__ void chunk_table(rsrc_t cr, rsrc_t sr, int c, int head_dim,
                                            float (&tc)[Vec<T>::N / 2],
                                            float (&ts)[Vec<T>::N / 2]) {
  constexpr int E = Vec<T>::N, PP = E / 2;
  const int hoff = (c * E) % head_dim;
  if constexpr (VEC) {
    load_tab<PP>(cr, hoff >> 1, tc);
    load_tab<PP>(sr, hoff >> 1, ts);
  } else {
#pragma unroll
    for (int p = 0; p < PP; ++p) {
      const int ho = (hoff + 2 * p) % head_dim;
      tc[p] = ld_f32(cr, (ho >> 1) * 4);
      ts[p] = ld_f32(sr, (ho >> 1) * 4);
    }
  }
}

// The per-element terms of one chunk: xhat, dy (rotated back for the RoPE
// epilogue, times gelu'(pre-activation) for the GeLU one) and g = dy w'.
template <typename T, bool LN, int EPI>
__device__ __forceinline__ void chunk_terms(const u32x4 xc, const u32x4 dc,
                                            const float (&wv)[Vec<T>::N],
                                            const float (&bv)[Vec<T>::N], float mu, float rs,
                                            const float (&tc)[Vec<T>::N / 2],
                                            const float (&ts)[Vec<T>::N / 2],
                                            float (&xh)[Vec<T>::N], float (&dd)[Vec<T>::N],
                                            float (&gg)[Vec<T>::N]) {
  constexpr int E = Vec<T>::N;
  float xv[E];
  unpack<T>(xc, xv);
  unpack<T>(dc, dd);
  if constexpr (EPI == kEpiRope) rotate_pairs<E / 2>(dd, tc, ts, -1.0f);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    xh[e] = (xv[e] - mu) * rs;
    if constexpr (EPI == kEpiGelu) dd[e] *= gelu_tanh_grad(fmaf(xh[e], wv[e], bv[e]));
    gg[e] = dd[e] * wv[e];
  }
}

// weights (w' and, for GeLU, beta) of chunk c, widened
template <typename T, bool VEC, int EPI>
__device__ __forceinline__ void chunk_weights(rsrc_t wr, rsrc_t br, bool have_w, float w_add, int c,
                                              float (&wv)[Vec<T>::N], float (&bv)[Vec<T>::N]) {
  constexpr int E = Vec<T>::N;
  unpack<T>(ld_chunk<T, VEC>(wr, c), wv);
#pragma unroll
  for (int e = 0; e < E; ++e) wv[e] = have_w ? wv[e] + w_add : 1.0f;
  if constexpr (EPI == kEpiGelu) {
    unpack<T>(ld_chunk<T, VEC>(br, c), bv);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) bv[e] = 0.0f;
  }
}

// Pass A: one 1024-thread workgroup per row; 4 chunks per lane in flight.
template <typename T, bool VEC, bool LN, int EPI>
__global__ void __launch_bounds__(1024)
norm_bwd_rowterms(const T* dy, const T* x, const T* w, const T* beta, const float* mean,
                  const float* rstat, float* terms, int n, float w_add, RopeArgs ra) {
  constexpr int E = Vec<T>::N, PP = E / 2, U = 4;
  constexpr bool ROPE = EPI == kEpiRope;
  __shared__ float red[2][16];
  const int t = threadIdx.x, nthr = blockDim.x;
  const int64_t row = blockIdx.x;
  const uint32_t rbytes = static_cast<uint32_t>(n) * sizeof(T);
  const int64_t off = row * static_cast<int64_t>(n);
  const rsrc_t xr = make_rsrc(x + off, rbytes);
  const rsrc_t gr = make_rsrc(dy + off, rbytes);
  const rsrc_t wr = make_rsrc(w, w != nullptr ? rbytes : 0u);
  const rsrc_t br = make_rsrc(beta, (EPI == kEpiGelu && beta != nullptr) ? rbytes : 0u);
  const int half = ra.head_dim >> 1;
  const int64_t tok = ROPE ? row / ra.rows_per_token : 0;
  const uint32_t tb = ROPE ? static_cast<uint32_t>(half) * 4u : 0u;
  const rsrc_t cr = make_rsrc(ra.cos_tab + tok * half, tb);
  const rsrc_t sr = make_rsrc(ra.sin_tab + tok * half, tb);
  const float rs = rstat[row];
  const float mu = LN ? mean[row] : 0.0f;
  const int nchunk = (n + E - 1) / E;

  float s1 = 0.0f, s2 = 0.0f;
  for (int c0 = t; c0 < nchunk; c0 += nthr * U) {
    u32x4 xc[U], dc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // chunks past the row read as 0 and add nothing
      xc[u] = ld_chunk<T, VEC, kStream>(xr, c0 + u * nthr);
      dc[u] = ld_chunk<T, VEC, kStream>(gr, c0 + u * nthr);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * nthr;
      float wv[E], bv[E], tc[PP], ts[PP], xh[E], dd[E], gg[E];
      chunk_weights<T, VEC, EPI>(wr, br, w != nullptr, w_add, c, wv, bv);
      if constexpr (ROPE) chunk_table<T, VEC>(cr, sr, c, ra.head_dim, tc, ts);
      chunk_terms<T, LN, EPI>(xc[u], dc[u], wv, bv, mu, rs, tc, ts, xh, dd, gg);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if constexpr (LN) {
          s1 += gg[e];
          s2 = fmaf(gg[e], xh[e], s2);
        } else {
          s1 = fmaf(gg[e], xh[e], s1);
        }
      }
    }
  }
  const int W = nthr >> 6, wave = wave_id();
  s1 = group_sum(s1, W, wave, 0, red[0]);
  if constexpr (LN) s2 = group_sum(s2, W, wave, 0, red[1]);
  if (t == 0) {
    const float inv_n = 1.0f / static_cast<float>(n);
    terms[2 * row] = s1 * inv_n;
    terms[2 * row + 1] = LN ? s2 * inv_n : 0.0f;
  }
}

// Pass B: workgroup (p, s) takes column slice s of rows p, p + P, ...
template <typename T, bool VEC, bool LN, int EPI>
__global__ void __launch_bounds__(kSplitLanes)
norm_bwd_colsplit(const T* dy, const T* x, const T* w, const T* beta, const float* mean,
                  const float* rstat, const float* terms, T* dx, float* part, int64_t part_stride,
                  int64_t rows, int n, float w_add, RopeArgs ra) {
  constexpr int E = Vec<T>::N, PP = E / 2, K = kSplitK;
  constexpr bool ROPE = EPI == kEpiRope;
  const int t = threadIdx.x;
  const int64_t P = gridDim.x;
  const int p = blockIdx.x;
  const int cbase = blockIdx.y * (kSplitLanes * K) + t;
  const uint32_t rbytes = static_cast<uint32_t>(n) * sizeof(T);
  const rsrc_t wr = make_rsrc(w, w != nullptr ? rbytes : 0u);
  const rsrc_t br = make_rsrc(beta, (EPI == kEpiGelu && beta != nullptr) ? rbytes : 0u);

  float wv[K][E], bv[K][E], acc1[K][E], acc2[K][E];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    chunk_weights<T, VEC, EPI>(wr, br, w != nullptr, w_add, cbase + k * kSplitLanes, wv[k], bv[k]);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      acc1[k][e] = 0.0f;
      acc2[k][e] = 0.0f;
    }
  }
  const int half = ra.head_dim >> 1;
  for (int64_t row = p; row < rows; row += P) {
    const int64_t off = row * static_cast<int64_t>(n);
    const rsrc_t xr = make_rsrc(x + off, rbytes);
    const rsrc_t gr = make_rsrc(dy + off, rbytes);
    const rsrc_t dr = make_rsrc(dx + off, rbytes);
    u32x4 xc[K], dc[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      xc[k] = ld_chunk<T, VEC, kStream>(xr, cbase + k * kSplitLanes);
      dc[k] = ld_chunk<T, VEC, kStream>(gr, cbase + k * kSplitLanes);
    }
    const float rs = rstat[row];
    const float mu = LN ? mean[row] : 0.0f;
    const float c1 = terms[2 * row], c2 = terms[2 * row + 1];
    const int64_t tok = ROPE ? row / ra.rows_per_token : 0;
    const uint32_t tb = ROPE ? static_cast<uint32_t>(half) * 4u : 0u;
    const rsrc_t cr = make_rsrc(ra.cos_tab + tok * half, tb);
    const rsrc_t sr = make_rsrc(ra.sin_tab + tok * half, tb);
    // LayerNorm: dx = r g - (r c1 + r c2 xhat); RMSNorm: dx = r (g - xhat c1)
    const float k1 = -rs * c1, k2 = -rs * c2;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int c = cbase + k * kSplitLanes;
      float tc[PP], ts[PP], xh[E], dd[E], gg[E], o[E];
      if constexpr (ROPE) chunk_table<T, VEC>(cr, sr, c, ra.head_dim, tc, ts);
      chunk_terms<T, LN, EPI>(xc[k], dc[k], wv[k], bv[k], mu, rs, tc, ts, xh, dd, gg);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        o[e] = LN ? fmaf(rs, gg[e], fmaf(xh[e], k2, k1)) : rs * fmaf(-xh[e], c1, gg[e]);
        acc1[k][e] = fmaf(dd[e], xh[e], acc1[k][e]);
        if constexpr (LN) acc2[k][e] += dd[e];
      }
      st_chunk<T, VEC, kStream>(dr, c, pack<T>(o));
    }
  }
  if (part != nullptr) {
    const uint32_t pbytes = static_cast<uint32_t>(n) * 4u;
    const rsrc_t p1 = make_rsrc(part + static_cast<int64_t>(p) * n, pbytes);
    const rsrc_t p2 = make_rsrc(part + part_stride + static_cast<int64_t>(p) * n, LN ? pbytes : 0u);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int c = cbase + k * kSplitLanes;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        st_f32(p1, (c * E + e) * 4, acc1[k][e]);
        if constexpr (LN) st_f32(p2, (c * E + e) * 4, acc2[k][e]);
      }
    }
  }
}

template <typename T, bool LN, int EPI>
hipError_t launch_bwd_long_t(bool aligned, const void* dy, const void* x, const void* w,
                             const void* beta, const float* mean, const float* rstat,
                             float* terms, void* dx, float* part, int64_t P, int64_t rows, int n,
                             float w_add, const RopeArgs& ra, hipStream_t st) {
  const int nchunk = (n + Vec<T>::N - 1) / Vec<T>::N;
  const unsigned slices = static_cast<unsigned>((nchunk + kSplitLanes * kSplitK - 1) /
                                                (kSplitLanes * kSplitK));
  const int64_t part_stride = P * n;
  auto a = aligned ? norm_bwd_rowterms<T, true, LN, EPI> : norm_bwd_rowterms<T, false, LN, EPI>;
  hipLaunchKernelGGL(a, dim3(static_cast<unsigned>(rows)), dim3(1024), 0, st,
                     static_cast<const T*>(dy), static_cast<const T*>(x), static_cast<const T*>(w),
                     static_cast<const T*>(beta), mean, rstat, terms, n, w_add, ra);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  auto b = aligned ? norm_bwd_colsplit<T, true, LN, EPI> : norm_bwd_colsplit<T, false, LN, EPI>;
  hipLaunchKernelGGL(b, dim3(static_cast<unsigned>(P), slices), dim3(kSplitLanes), 0, st,
                     static_cast<const T*>(dy), static_cast<const T*>(x), static_cast<const T*>(w),
                     static_cast<const T*>(beta), mean, rstat, terms, static_cast<T*>(dx), part,
                     part_stride, rows, n, w_add, ra);
  return hipGetLastError();
}

#define NR_BWD_LONG_INSTANTIATE(T, LN, EPI)                                                   \
  template hipError_t launch_bwd_long_t<T, LN, EPI>(bool, const void*, const void*, const void*, \
                                                    const void*, const float*, const float*,    \
                                                    float*, void*, float*, int64_t, int64_t, int, \
                                                    float, const RopeArgs&, hipStream_t);

}  // namespace nr
