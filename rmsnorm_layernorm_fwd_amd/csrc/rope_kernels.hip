// rope_kernels.hip -- in-place interleaved rotary position embedding for
// gfx950, forward and inverse, and the cos/sin table builders.
//
// Operation (Helios 性能优化全解析, 内核二 FlashRoPE): the frequencies are laid
// out even/odd interleaved, so element 2i of a head vector is the real part
// and element 2i+1 the imaginary part of pair i.  Each pair is rotated by its
// token's angle and written back to where it was read, with no intermediate
// tensor.  The inverse (which is also the backward, a rotation's transpose
// being its inverse) is the same kernel with sin negated.
//
// Mapping: `groups` wavefronts per token (the host picks about 4 chunks per
// lane per wave).  The token's H head vectors of D elements are cut into
// 16-byte chunks (4 bf16 pairs or 2 fp32 pairs); lane l of the token's wave
// g owns chunks 64 K g + l, + 64, ..., so each wave-wide load covers 1 KiB
// of contiguous memory when heads are packed.  When 64 is a multiple of the
// chunks per head (D = 128 bf16: 16 chunks), a lane always lands on the same
// pair slot of every head it visits, so it fetches its cos/sin slice of the
// token's table row once and reuses it for all heads.  Every element is read
// and written by the same lane, so the in-place update has no hazard.
#include "nr_device.hpp"
#include "nr_internal.hpp"

namespace nr {

// byte offset handed to lanes that own no chunk: beyond every token span the
// host accepts, so their loads read 0 and their stores are dropped
constexpr int kNoChunk = 0x7ffffff0;

template <typename T, int K, bool VEC, bool FAST>
__global__ void __launch_bounds__(256)
rope_apply_kernel(T* x, const float* cos_tab, const float* sin_tab, int64_t ntok,
                  int64_t tokens, int heads, int head_dim, int64_t sb, int64_t stok,
                  int64_t sh, uint32_t span_bytes, float sign, int groups) {
  constexpr int E = VEC ? Vec<T>::N : 2;  // elements per chunk
  constexpr int PP = E / 2;               // pairs per chunk
  const int lane = threadIdx.x & 63;
  // `groups` waves share a token: wave g of it starts at chunk 64 K g and
  // steps by 64 K groups
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + wave_id();
  const int64_t tok = gw / groups;
  const int grp = static_cast<int>(gw - tok * groups);
  if (tok >= ntok) return;  // whole wave; no barrier below
  const int64_t bi = tok / tokens;
  const int64_t s = tok - bi * tokens;
  const int half = head_dim >> 1;
  const rsrc_t xr = make_rsrc(x + bi * sb + s * stok, span_bytes);
  const rsrc_t cr = make_rsrc(cos_tab + s * half, static_cast<uint32_t>(half) * 4u);
  const rsrc_t sr = make_rsrc(sin_tab + s * half, static_cast<uint32_t>(half) * 4u);
  const int cph = head_dim / E;
  const int nchunk = heads * cph;

  float cf[PP], sf[PP];
  if constexpr (FAST) {
    const int c = lane % cph;
    load_tab<PP>(cr, c * PP, cf);
    load_tab<PP>(sr, c * PP, sf);
  }

  for (int c0 = 64 * K * grp; c0 < nchunk; c0 += 64 * K * groups) {
    float v[K][E];
    float ck[K][PP], sk[K][PP];
    int off[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int idx = c0 + lane + 64 * k;
      const int h = idx / cph;
      const int c = idx - h * cph;
      off[k] = idx < nchunk ? static_cast<int>((h * sh + c * E) * static_cast<int64_t>(sizeof(T)))
                            : kNoChunk;
      if constexpr (VEC) {
        unpack<T>(__builtin_amdgcn_raw_buffer_load_b128(xr, off[k], 0, kStream), v[k]);
      } else {
        v[k][0] = ld_elem<T>(xr, off[k]);
        v[k][1] = ld_elem<T>(xr, off[k] + static_cast<int>(sizeof(T)));
      }
      if constexpr (!FAST) {
        load_tab<PP>(cr, c * PP, ck[k]);
        load_tab<PP>(sr, c * PP, sk[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if constexpr (FAST) {
        rotate_pairs<PP>(v[k], cf, sf, sign);
      } else {
        rotate_pairs<PP>(v[k], ck[k], sk[k], sign);
      }
      if constexpr (VEC) {
        __builtin_amdgcn_raw_buffer_store_b128(pack<T>(v[k]), xr, off[k], 0, kStreamStore);
      } else {
        st_elem<T>(xr, off[k], v[k][0]);
        st_elem<T>(xr, off[k] + static_cast<int>(sizeof(T)), v[k][1]);
      }
    }
  }
}

// Table builders: angle = position x frequency in double precision (a 65536
// token position times a unit frequency must not lose bits before cos/sin),
// then cos and sin rounded once to fp32.  Layout [tokens][head_dim / 2].
__global__ void rope_table_1d_kernel(float* cos_tab, float* sin_tab, int64_t total, int half,
                                     int head_dim, int64_t pos0, double log2_theta) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int64_t s = idx / half;
  const int i = static_cast<int>(idx - s * half);
  const double freq = exp2(-2.0 * i / head_dim * log2_theta);
  double sv, cv;
  sincos(static_cast<double>(pos0 + s) * freq, &sv, &cv);
  cos_tab[idx] = static_cast<float>(cv);
  sin_tab[idx] = static_cast<float>(sv);
}

// 3-D grid: token s = (f * H + h) * W + w; the first pt pairs follow f, the
// next ph follow h, the last pw follow w; an axis with P pairs uses the
// frequencies of a P-pair (2P-dimensional) 1-D table.
__global__ void rope_table_3d_kernel(float* cos_tab, float* sin_tab, int64_t total, int64_t height,
                                     int64_t width, int pt, int ph, int pw, double log2_theta) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int half = pt + ph + pw;
  const int64_t s = idx / half;
  const int i = static_cast<int>(idx - s * half);
  const int64_t hw = height * width;
  const int64_t f = s / hw;
  const int64_t rem = s - f * hw;
  const int64_t h = rem / width;
  const int64_t w = rem - h * width;
  int64_t pos;
  int j, np;
  if (i < pt) {
    pos = f, j = i, np = pt;
  } else if (i < pt + ph) {
    pos = h, j = i - pt, np = ph;
  } else {
    pos = w, j = i - pt - ph, np = pw;
  }
  const double freq = exp2(-2.0 * j / (2.0 * np) * log2_theta);
  double sv, cv;
  sincos(static_cast<double>(pos) * freq, &sv, &cv);
  cos_tab[idx] = static_cast<float>(cv);
  sin_tab[idx] = static_cast<float>(sv);
}

namespace {

template <typename T, int K, bool A, bool F>
hipError_t launch_rope_kaf(const RopePlan& pl, void* x, const float* ct, const float* stb,
                           int64_t batch, int64_t tokens, int heads, int head_dim, int64_t sb,
                           int64_t stok, int64_t sh, float sign, hipStream_t st) {
  const int64_t ntok = batch * tokens;
  const uint32_t span = static_cast<uint32_t>(((heads - 1) * sh + head_dim) * static_cast<int64_t>(sizeof(T)));
  const int64_t waves = ntok * pl.groups;
  const dim3 grid(static_cast<unsigned>((waves + pl.waves_per_block - 1) / pl.waves_per_block));
  hipLaunchKernelGGL((rope_apply_kernel<T, K, A, F>), grid, dim3(64 * pl.waves_per_block), 0, st,
                     static_cast<T*>(x), ct, stb, ntok, tokens, heads, head_dim, sb, stok, sh,
                     span, sign, pl.groups);
  return hipGetLastError();
}

template <typename T, int K>
hipError_t launch_rope_k(const RopePlan& pl, void* x, const float* ct, const float* stb,
                         int64_t batch, int64_t tokens, int heads, int head_dim, int64_t sb,
                         int64_t stok, int64_t sh, float sign, hipStream_t st) {
  if (pl.aligned) {
    return pl.fast ? launch_rope_kaf<T, K, true, true>(pl, x, ct, stb, batch, tokens, heads, head_dim, sb, stok, sh, sign, st)
                   : launch_rope_kaf<T, K, true, false>(pl, x, ct, stb, batch, tokens, heads, head_dim, sb, stok, sh, sign, st);
  }
  return pl.fast ? launch_rope_kaf<T, K, false, true>(pl, x, ct, stb, batch, tokens, heads, head_dim, sb, stok, sh, sign, st)
                 : launch_rope_kaf<T, K, false, false>(pl, x, ct, stb, batch, tokens, heads, head_dim, sb, stok, sh, sign, st);
}

template <typename T>
hipError_t launch_rope_t(const RopePlan& pl, void* x, const float* ct, const float* stb,
                         int64_t batch, int64_t tokens, int heads, int head_dim, int64_t sb,
                         int64_t stok, int64_t sh, float sign, hipStream_t st) {
  switch (pl.K) {
#define NR_CASE(KK) \
  case KK: return launch_rope_k<T, KK>(pl, x, ct, stb, batch, tokens, heads, head_dim, sb, stok, sh, sign, st);
    NR_CASE(1) NR_CASE(2) NR_CASE(4) NR_CASE(5) NR_CASE(6) NR_CASE(8) NR_CASE(10)
#undef NR_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_rope(int dt, const RopePlan& pl, void* x, const float* cos_tab,
                       const float* sin_tab, int64_t batch, int64_t tokens, int heads,
                       int head_dim, int64_t sb, int64_t stok, int64_t sh, float sign,
                       hipStream_t st) {
  return by_dtype(dt, [&](auto tag) {
    return launch_rope_t<decltype(tag)>(pl, x, cos_tab, sin_tab, batch, tokens, heads, head_dim, sb,
                                        stok, sh, sign, st);
  });
}

hipError_t launch_rope_table_1d(float* cos_tab, float* sin_tab, int64_t tokens, int head_dim,
                                int64_t pos0, double theta, hipStream_t st) {
  const int half = head_dim / 2;
  const int64_t total = tokens * half;
  const unsigned blocks = static_cast<unsigned>((total + 255) / 256);
  hipLaunchKernelGGL(rope_table_1d_kernel, dim3(blocks), dim3(256), 0, st, cos_tab, sin_tab,
                     total, half, head_dim, pos0, log2(theta));
  return hipGetLastError();
}

hipError_t launch_rope_table_3d(float* cos_tab, float* sin_tab, int64_t frames, int64_t height,
                                int64_t width, int pt, int ph, int pw, double theta,
                                hipStream_t st) {
  const int64_t total = frames * height * width * (pt + ph + pw);
  const unsigned blocks = static_cast<unsigned>((total + 255) / 256);
  hipLaunchKernelGGL(rope_table_3d_kernel, dim3(blocks), dim3(256), 0, st, cos_tab, sin_tab,
                     total, height, width, pt, ph, pw, log2(theta));
  return hipGetLastError();
}

}  // namespace nr
