// norm_fwd_packed.hip -- RMSNorm / LayerNorm forward of short rows, several
// rows to a wavefront.
//
// Operation: as the row kernels of norm_fwd.hpp (Helios 性能优化全解析,
// 内核一 FlashNorm: one read of the row, its sums on chip, one write of the
// normalised and weighted row, the per-row statistics kept for the backward;
// fp32 arithmetic and a single rounding per output, Janus-Pro-7B模型推理加速
// 实战, 3. 计算精度优化), with the same epilogues (RoPE after RMSNorm,
// tanh-GeLU after LayerNorm).
//
// Mapping: a row of at most 32 whole 16-byte chunks (256 bf16 / fp16 or 128
// fp32 elements: a per-head q/k norm, a small hidden size) takes S lanes of
// a wave, S the power of two >= its chunk count (at least 4); lane c of the
// S owns chunk c.  A wave holds 64 / S rows side by side and PJ such groups
// one after the other, all loaded before the first is used: PJ x 16 bytes in
// flight per lane, every lane busy, where a wave per row would leave most of
// its lanes idle on these rows.  The consecutive rows of a wave are one
// contiguous span of memory, so each load instruction covers 64 / S whole
// rows.  Row sums are butterflies inside the S lanes (DPP inside a 16-lane
// row, v_permlane16_swap across two rows), so every lane of a row gets the
// same bits and there is no LDS and no barrier.
#include "nr_device.hpp"
#include "nr_internal.hpp"

#ifndef NR_PACK_J
#define NR_PACK_J 4
#endif

namespace nr {

namespace {

constexpr int PJ = NR_PACK_J;  // row groups a wave loads at once

}  // namespace

template <typename T, int S, bool LN, int EPI>
__global__ __launch_bounds__(256) void norm_fwd_packed(const T* __restrict__ x,
                                                       const T* __restrict__ w,
                                                       const T* __restrict__ b, T* __restrict__ y,
                                                       float* __restrict__ stat0,
                                                       float* __restrict__ stat1, int64_t rows,
                                                       int n, float eps, float w_add,
                                                       RopeArgs ra) {
  constexpr int E = Vec<T>::N;
  constexpr int L = 64 / S;  // rows side by side in a wave
  constexpr bool ROPE = EPI == kEpiRope;
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int slot = lane / S;
  const int c = lane % S;
  const int64_t base =
      (static_cast<int64_t>(blockIdx.x) * 4 + (static_cast<int>(threadIdx.x) >> 6)) * (PJ * L);
  if (base >= rows) return;  // whole waves only; the kernel has no barrier
  const int64_t left = rows - base;
  const int nw = left < PJ * L ? static_cast<int>(left) : PJ * L;  // rows of this wave
  const uint32_t rb = static_cast<uint32_t>(n) * sizeof(T);
  const uint32_t span = static_cast<uint32_t>(nw) * rb;
  const rsrc_t xr = make_rsrc(x + base * n, span);
  const rsrc_t yr = make_rsrc(y + base * n, span);
  // lanes past the row's chunks point at the end of the span: their loads
  // return 0 and their stores are dropped, as for rows past the last one
  const bool has = c * E < n;
  uint32_t off[PJ];
#pragma unroll
  for (int j = 0; j < PJ; ++j)
    off[j] = has ? static_cast<uint32_t>(j * L + slot) * rb + static_cast<uint32_t>(c) * 16u : span;

  u32x4 xa[PJ], wa, ba;
#pragma unroll
  for (int j = 0; j < PJ; ++j)
    xa[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, static_cast<int>(off[j]), 0, kStream);
  {
    // chunk c of a weight lies past its end exactly when the lane has no chunk
    const rsrc_t wr = make_rsrc(w, w != nullptr ? rb : 0u);
    wa = ld_chunk<T, true>(wr, c);
    if constexpr (LN) {
      const rsrc_t br = make_rsrc(b, b != nullptr ? rb : 0u);
      ba = ld_chunk<T, true>(br, c);
    }
  }

  const float fn = static_cast<float>(n);
  const float wadd = (w != nullptr) ? w_add : 1.0f;
  float mean[PJ], r[PJ];
  if constexpr (LN) {
    float s[PJ];
#pragma unroll
    for (int j = 0; j < PJ; ++j) {
      float v[E];
      unpack<T>(xa[j], v);
      s[j] = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) s[j] += v[e];
    }
#pragma unroll
    for (int j = 0; j < PJ; ++j) s[j] = lane_group_sum<S>(s[j]);
    float q[PJ];
#pragma unroll
    for (int j = 0; j < PJ; ++j) {
      mean[j] = s[j] / fn;
      float v[E];
      unpack<T>(xa[j], v);
      q[j] = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float d = has ? v[e] - mean[j] : 0.0f;  // a chunk is wholly in or out
        q[j] = fmaf(d, d, q[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < PJ; ++j) r[j] = rsqrtf(lane_group_sum<S>(q[j]) / fn + eps);
  } else {
    float ss[PJ];
#pragma unroll
    for (int j = 0; j < PJ; ++j) {
      float v[E];
      unpack<T>(xa[j], v);
      ss[j] = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) ss[j] = fmaf(v[e], v[e], ss[j]);
    }
#pragma unroll
    for (int j = 0; j < PJ; ++j) {
      mean[j] = 0.0f;
      r[j] = rsqrtf(lane_group_sum<S>(ss[j]) / fn + eps);
    }
  }

  // RoPE: the table rows of the wave's tokens, from the first one on; this
  // lane's chunk starts at element hoff of its head (whole chunks lie inside
  // one head)
  const int half = ra.head_dim >> 1;
  const int hoff = ROPE ? (c * E) % ra.head_dim : 0;
  const int64_t tok0 = ROPE ? base / ra.rows_per_token : 0;
  const uint32_t tb =
      ROPE ? static_cast<uint32_t>(((base + nw - 1) / ra.rows_per_token + 1 - tok0) * half * 4) : 0u;
  const rsrc_t cr = make_rsrc(ROPE ? ra.cos_tab + tok0 * half : nullptr, tb);
  const rsrc_t sr = make_rsrc(ROPE ? ra.sin_tab + tok0 * half : nullptr, tb);

  float wv[E], bv[E];
  unpack<T>(wa, wv);
  if constexpr (LN) unpack<T>(ba, bv);
#pragma unroll
  for (int j = 0; j < PJ; ++j) {
    const int64_t row = base + j * L + slot;
    float v[E], o[E];
    unpack<T>(xa[j], v);
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
      const int64_t tok = (row < rows ? row : base) / ra.rows_per_token;
      const int e0 = static_cast<int>((tok - tok0) * half) + (hoff >> 1);
      float cf[PP], sf[PP];
      load_tab<PP>(cr, e0, cf);
      load_tab<PP>(sr, e0, sf);
      rotate_pairs<PP>(o, cf, sf, 1.0f);
    }
    __builtin_amdgcn_raw_buffer_store_b128(pack<T>(o), yr, static_cast<int>(off[j]), 0, kNormStore);
    if (c == 0 && j * L + slot < nw) {
      if constexpr (LN) {
        if (stat0) stat0[row] = mean[j];
        if (stat1) stat1[row] = r[j];
      } else {
        if (stat0) stat0[row] = r[j];
      }
    }
  }
}

int fwd_packed_rows_per_block(int S) { return 4 * PJ * (64 / S); }

namespace {

template <typename T, int S, bool LN, int EPI>
hipError_t launch_packed(const void* x, const void* w, const void* b, void* y, float* s0,
                         float* s1, int64_t rows, int n, float eps, float w_add,
                         const RopeArgs& ra, hipStream_t st) {
  const int64_t per_block = fwd_packed_rows_per_block(S);
  const dim3 grid(static_cast<unsigned>((rows + per_block - 1) / per_block));
  hipLaunchKernelGGL((norm_fwd_packed<T, S, LN, EPI>), grid, dim3(256), 0, st,
                     static_cast<const T*>(x), static_cast<const T*>(w), static_cast<const T*>(b),
                     static_cast<T*>(y), s0, s1, rows, n, eps, w_add, ra);
  return hipGetLastError();
}

template <typename T, bool LN, int EPI>
hipError_t launch_packed_s(int S, const void* x, const void* w, const void* b, void* y, float* s0,
                           float* s1, int64_t rows, int n, float eps, float w_add,
                           const RopeArgs& ra, hipStream_t st) {
  switch (S) {
    case 4: return launch_packed<T, 4, LN, EPI>(x, w, b, y, s0, s1, rows, n, eps, w_add, ra, st);
    case 8: return launch_packed<T, 8, LN, EPI>(x, w, b, y, s0, s1, rows, n, eps, w_add, ra, st);
    case 16: return launch_packed<T, 16, LN, EPI>(x, w, b, y, s0, s1, rows, n, eps, w_add, ra, st);
    case 32: return launch_packed<T, 32, LN, EPI>(x, w, b, y, s0, s1, rows, n, eps, w_add, ra, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fwd_packed(int dt, bool ln, int epi, const FwdPlan& pl, const void* x,
                             const void* w, const void* b, void* y, float* s0, float* s1,
                             int64_t rows, int n, float eps, float w_add, const RopeArgs& ra,
                             hipStream_t st) {
  // the planner packs only whole 16-byte chunks, at most S of them a row
  if (!pl.aligned || n > pl.S * (dt == 0 ? 4 : 8)) return hipErrorInvalidValue;
  return by_dtype(dt, [&](auto tag) {
    using T = decltype(tag);
    if (epi == kEpiRope) {
      if (ln) return hipErrorInvalidValue;
      return launch_packed_s<T, false, kEpiRope>(pl.S, x, w, b, y, s0, s1, rows, n, eps, w_add, ra, st);
    }
    if (epi == kEpiGelu) {
      if (!ln) return hipErrorInvalidValue;
      return launch_packed_s<T, true, kEpiGelu>(pl.S, x, w, b, y, s0, s1, rows, n, eps, w_add, ra, st);
    }
    return ln ? launch_packed_s<T, true, kEpiNone>(pl.S, x, w, b, y, s0, s1, rows, n, eps, w_add, ra, st)
              : launch_packed_s<T, false, kEpiNone>(pl.S, x, w, b, y, s0, s1, rows, n, eps, w_add, ra, st);
  });
}

}  // namespace nr
