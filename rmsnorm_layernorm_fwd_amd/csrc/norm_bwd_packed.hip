// norm_bwd_packed.hip -- RMSNorm / LayerNorm backward of short rows, several
// rows to a wavefront, stage 1 of the two-stage column reduction.
//
// Operation (Helios 性能优化全解析, 内核一 FlashNorm, and the backward of
// the same norm): with x^ the normalised row, r its inverse root and g = dy w'
// (w' = w, 1 + w for the Gemma variant, or 1), RMSNorm's dx = r (g - x^
// mean(g x^)) and LayerNorm's dx = r (g - mean(g) - x^ mean(g x^)); the
// weight gradients are column sums over the rows, dw = sum dy x^ (and
// dbeta = sum dy).  After RoPE the incoming gradient is first rotated back
// by the token's angles; after LayerNorm + tanh-GeLU (LLM层的优化算子,
// 编写定制融合算子) it is first multiplied by the activation's derivative at
// x^ gamma + beta.  fp32 arithmetic, one rounding per output.
//
// Mapping as the packed forward (norm_fwd_packed.hip): a row of at most 32
// whole 16-byte chunks takes S lanes of a wave, 64 / S rows side by side and
// PJ such groups per batch of the wave.  P workgroups of four waves take the
// batches round-robin (wave i of the grid: batches i, i + 4P, ...).  Each lane
// keeps its chunk's column sums over the rows it saw; at the end the
// workgroup adds the 4 x (64 / S) lanes that share a chunk in a fixed order
// through LDS and writes one partial row, which colreduce then sums over the
// P workgroups in a fixed order: bitwise reproducible for a given shape.
#include "nr_device.hpp"
#include "nr_internal.hpp"

#ifndef NR_PACK_BWD_J
#define NR_PACK_BWD_J 4
#endif

namespace nr {

namespace {

constexpr int PJB = NR_PACK_BWD_J;  // row groups a wave loads per batch

}  // namespace

template <typename T, int S, bool LN, int EPI>
__global__ __launch_bounds__(256) void norm_bwd_packed(
    const T* __restrict__ dy, const T* __restrict__ x, const T* __restrict__ w,
    const T* __restrict__ b, const float* __restrict__ mean, const float* __restrict__ rstat, T* __restrict__ dx,
    float* __restrict__ part, int64_t rows, int n, float w_add, RopeArgs ra) {
  constexpr int E = Vec<T>::N;
  constexpr int L = 64 / S;      // rows side by side in a wave
  constexpr int RW = PJB * L;    // rows per batch of a wave
  constexpr int NA = LN ? 2 : 1;  // column sums per element
  constexpr bool ROPE = EPI == kEpiRope;
  constexpr bool GELU = EPI == kEpiGelu;
  constexpr bool PRE = ROPE || GELU;  // the incoming gradient transformed first
  __shared__ float red[NA * 256 * E];
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int wave = static_cast<int>(threadIdx.x) >> 6;
  const int slot = lane / S;
  const int c = lane % S;
  const bool has = c * E < n;
  const uint32_t rb = static_cast<uint32_t>(n) * sizeof(T);
  const float inv_n = 1.0f / static_cast<float>(n);

  float wv[E];
  {
    const rsrc_t wr = make_rsrc(w, w != nullptr ? rb : 0u);
    unpack<T>(ld_chunk<T, true>(wr, c), wv);
    const float wadd = (w != nullptr) ? w_add : 1.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) wv[e] += wadd;
  }
  float bv[GELU ? E : 1];
  if constexpr (GELU) {
    const rsrc_t br = make_rsrc(b, b != nullptr ? rb : 0u);
    unpack<T>(ld_chunk<T, true>(br, c), bv);
  }
  float acc[NA][E];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[a][e] = 0.0f;

  const int half = ra.head_dim >> 1;
  const int hoff = ROPE ? (c * E) % ra.head_dim : 0;
  const int64_t nb = (rows + RW - 1) / RW;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 4;
  for (int64_t bi = static_cast<int64_t>(blockIdx.x) * 4 + wave; bi < nb; bi += stride) {
    const int64_t base = bi * RW;
    const int64_t left = rows - base;
    const int nw = left < RW ? static_cast<int>(left) : RW;
    const uint32_t span = static_cast<uint32_t>(nw) * rb;
    const rsrc_t dyr = make_rsrc(dy + base * n, span);
    const rsrc_t xr = make_rsrc(x + base * n, span);
    const rsrc_t dxr = make_rsrc(dx + base * n, span);
    const rsrc_t rr = make_rsrc(rstat + base, static_cast<uint32_t>(nw) * 4u);
    const rsrc_t mr = make_rsrc(LN ? mean + base : nullptr, LN ? static_cast<uint32_t>(nw) * 4u : 0u);
    uint32_t off[PJB];
    u32x4 xa[PJB], da[PJB];
    float rs[PJB], mu[PJB];
#pragma unroll
    for (int j = 0; j < PJB; ++j) {
      // lanes past the row's chunks point at the end of the span (loads 0,
      // stores dropped), as do rows past the last one
      off[j] = has ? static_cast<uint32_t>(j * L + slot) * rb + static_cast<uint32_t>(c) * 16u : span;
      da[j] = __builtin_amdgcn_raw_buffer_load_b128(dyr, static_cast<int>(off[j]), 0, kStream);
      xa[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, static_cast<int>(off[j]), 0, kStream);
      rs[j] = ld_f32(rr, (j * L + slot) * 4);
      mu[j] = LN ? ld_f32(mr, (j * L + slot) * 4) : 0.0f;
    }
    // RoPE: the incoming gradient rotated back by its token's angles; GeLU:
    // times the derivative at the pre-activation
    float dr[PRE ? PJB : 1][E];
    if constexpr (GELU) {
#pragma unroll
      for (int j = 0; j < PJB; ++j) {
        float xv[E];
        unpack<T>(xa[j], xv);
        unpack<T>(da[j], dr[j]);
#pragma unroll
        for (int e = 0; e < E; ++e)
          dr[j][e] *= gelu_tanh_grad(fmaf((xv[e] - mu[j]) * rs[j], wv[e], bv[e]));
      }
    }
    if constexpr (ROPE) {
      constexpr int PP = E / 2;
      const int64_t tok0 = base / ra.rows_per_token;
      const uint32_t tb =
          static_cast<uint32_t>(((base + nw - 1) / ra.rows_per_token + 1 - tok0) * half * 4);
      const rsrc_t cr = make_rsrc(ra.cos_tab + tok0 * half, tb);
      const rsrc_t sr = make_rsrc(ra.sin_tab + tok0 * half, tb);
#pragma unroll
      for (int j = 0; j < PJB; ++j) {
        const int64_t row = base + j * L + slot;
        const int64_t tok = (row < rows ? row : base) / ra.rows_per_token;
        const int e0 = static_cast<int>((tok - tok0) * half) + (hoff >> 1);
        float cf[PP], sf[PP];
        load_tab<PP>(cr, e0, cf);
        load_tab<PP>(sr, e0, sf);
        unpack<T>(da[j], dr[j]);
        rotate_pairs<PP>(dr[j], cf, sf, -1.0f);
      }
    }
    // the row sums: sum g x^ (and sum g for LayerNorm)
    float s1[PJB], s2[PJB];
#pragma unroll
    for (int j = 0; j < PJB; ++j) {
      float xv[E], dv[E];
      unpack<T>(xa[j], xv);
      if constexpr (PRE) {
#pragma unroll
        for (int e = 0; e < E; ++e) dv[e] = dr[j][e];
      } else {
        unpack<T>(da[j], dv);
      }
      s1[j] = 0.0f;
      s2[j] = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float gg = dv[e] * wv[e];
        const float xh = (xv[e] - mu[j]) * rs[j];
        if constexpr (LN) {
          s1[j] += gg;
          s2[j] = fmaf(gg, xh, s2[j]);
        } else {
          s1[j] = fmaf(gg, xh, s1[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < PJB; ++j) {
      s1[j] = lane_group_sum<S>(s1[j]);
      if constexpr (LN) s2[j] = lane_group_sum<S>(s2[j]);
    }
    // widen the packed chunks again after the sums rather than keep their
    // fp32 copies alive across them
    reload_barrier<PJB>(xa);
    if constexpr (!PRE) reload_barrier<PJB>(da);
#pragma unroll
    for (int j = 0; j < PJB; ++j) {
      float xv[E], dv[E], o[E];
      unpack<T>(xa[j], xv);
      if constexpr (PRE) {
#pragma unroll
        for (int e = 0; e < E; ++e) dv[e] = dr[j][e];
      } else {
        unpack<T>(da[j], dv);
      }
      const float c1 = s1[j] * inv_n;
      const float c2 = LN ? s2[j] * inv_n : 0.0f;
      const float k1 = -rs[j] * c1, k2 = -rs[j] * c2;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float gg = dv[e] * wv[e];
        const float xh = (xv[e] - mu[j]) * rs[j];
        if constexpr (LN) {
          o[e] = fmaf(rs[j], gg, fmaf(xh, k2, k1));
          acc[1][e] += dv[e];
        } else {
          o[e] = rs[j] * (gg - xh * c1);
        }
        acc[0][e] = fmaf(dv[e], xh, acc[0][e]);
      }
      __builtin_amdgcn_raw_buffer_store_b128(pack<T>(o), dxr, static_cast<int>(off[j]), 0, kNormStore);
    }
  }

  if (part == nullptr) return;  // uniform: no column gradients asked for
  // the 4 L lanes that hold chunk c: in LDS, then added in (wave, slot) order
  const int q = wave * L + slot;
  if (has) {
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int e = 0; e < E; ++e) red[(a * 4 * L + q) * (S * E) + c * E + e] = acc[a][e];
  }
  __syncthreads();
  const int64_t P = gridDim.x;
  for (int col = static_cast<int>(threadIdx.x); col < n; col += 256) {
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      float t = 0.0f;
      for (int i = 0; i < 4 * L; ++i) t += red[(a * 4 * L + i) * (S * E) + col];
      part[(a * P + blockIdx.x) * static_cast<int64_t>(n) + col] = t;
    }
  }
}

namespace {

template <typename T, int S, bool LN, int EPI>
hipError_t launch_bwd_packed_s(int P, const void* dy, const void* x, const void* w,
                               const void* b, const float* mean, const float* rstat, void* dx, float* part,
                               int64_t rows, int n, float w_add, const RopeArgs& ra,
                               hipStream_t st) {
  hipLaunchKernelGGL((norm_bwd_packed<T, S, LN, EPI>), dim3(P), dim3(256), 0, st,
                     static_cast<const T*>(dy), static_cast<const T*>(x),
                     static_cast<const T*>(w), static_cast<const T*>(b), mean, rstat, static_cast<T*>(dx), part, rows, n,
                     w_add, ra);
  return hipGetLastError();
}

template <typename T, bool LN, int EPI>
hipError_t launch_bwd_packed_t(int S, int P, const void* dy, const void* x, const void* w,
                               const void* b, const float* mean, const float* rstat, void* dx, float* part,
                               int64_t rows, int n, float w_add, const RopeArgs& ra,
                               hipStream_t st) {
  switch (S) {
#define NR_CASE(SS)                                                                              \
  case SS:                                                                                       \
    return launch_bwd_packed_s<T, SS, LN, EPI>(P, dy, x, w, b, mean, rstat, dx, part, rows, n,  \
                                                w_add, ra, st);
    NR_CASE(4) NR_CASE(8) NR_CASE(16) NR_CASE(32)
#undef NR_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int bwd_packed_rows_per_wave(int S) { return PJB * (64 / S); }

hipError_t launch_bwd_packed(int dt, bool ln, int epi, int S, int P, const void* dy,
                             const void* x, const void* w, const void* b, const float* mean,
                             const float* rstat, void* dx, float* part, int64_t rows, int n,
                             float w_add, const RopeArgs& ra, hipStream_t st) {
  // whole 16-byte chunks only, at most S of them a row; RoPE after RMSNorm,
  // GeLU after LayerNorm
  if (P < 1 || n > S * (dt == 0 ? 4 : 8) || (epi == kEpiRope && ln) || (epi == kEpiGelu && !ln))
    return hipErrorInvalidValue;
  return by_dtype(dt, [&](auto tag) {
    using T = decltype(tag);
    if (epi == kEpiRope)
      return launch_bwd_packed_t<T, false, kEpiRope>(S, P, dy, x, w, b, mean, rstat, dx, part,
                                                     rows, n, w_add, ra, st);
    if (epi == kEpiGelu)
      return launch_bwd_packed_t<T, true, kEpiGelu>(S, P, dy, x, w, b, mean, rstat, dx, part,
                                                    rows, n, w_add, ra, st);
    return ln ? launch_bwd_packed_t<T, true, kEpiNone>(S, P, dy, x, w, b, mean, rstat, dx, part,
                                                       rows, n, w_add, ra, st)
              : launch_bwd_packed_t<T, false, kEpiNone>(S, P, dy, x, w, b, mean, rstat, dx, part,
                                                        rows, n, w_add, ra, st);
  });
}

}  // namespace nr
