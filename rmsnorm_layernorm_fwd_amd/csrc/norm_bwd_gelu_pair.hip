// norm_bwd_gelu_pair.hip -- LayerNorm + tanh-GeLU backward (stage 1) for
// 16-bit rows of 640 W elements, W = 4 or 8 (2560 and 5120 elements).
//
// Same operation, order of work and column partials as norm_bwd_rows with the
// GeLU epilogue (the fused example of "LLM层的优化算子", 编写定制融合算子;
// statistics cached by the forward, Helios 性能优化全解析, 内核一 FlashNorm),
// on a different lane geometry.  That kernel is VALU-bound: with one 16-byte
// chunk (8 elements) a lane a 5120-wide row takes 10 waves, which sit 3/3/2/2
// on the CU's four SIMDs, and the two fuller SIMDs set each row's pace (per-row
// time follows the most waves on one SIMD: 77 us for 15360 rows of 4096 on 8
// waves, 94 us for 5120 on 10, 103 us for 6144 on 12).  Here each lane owns 10
// elements -- its 16-byte chunk t in the first 512 W elements and the
// 2-element pair t in the last 128 W -- so the row takes W = n / 640 waves, the
// same number on every SIMD.
#include "nr_device.hpp"
#include "nr_internal.hpp"

namespace nr {

namespace {

constexpr int kPairElems = 10;  // elements a lane: a chunk of 8 and a pair

// one row of x and dout as loaded (packed), and its statistics (uniform)
struct PairBatch {
  u32x4 xc, gc;     // the lane's 16-byte chunk of x and of dout
  uint32_t xp, gp;  // its 2-element pair
  float rs, mu;
};

template <typename T>
__device__ __forceinline__ void unpack2(uint32_t word, float* v);
template <>
__device__ __forceinline__ void unpack2<bf16>(uint32_t word, float* v) {
  v[0] = __uint_as_float(word << 16);
  v[1] = __uint_as_float(word & 0xffff0000u);
}
template <>
__device__ __forceinline__ void unpack2<f16>(uint32_t word, float* v) {
  const f32x2 f = __builtin_convertvector(__builtin_bit_cast(f16x2, word), f32x2);
  v[0] = f[0];
  v[1] = f[1];
}

template <typename T>
__device__ __forceinline__ uint32_t pack2(float a, float b);
template <>
__device__ __forceinline__ uint32_t pack2<bf16>(float a, float b) {
  return pack_bf16x2(a, b);
}
template <>
__device__ __forceinline__ uint32_t pack2<f16>(float a, float b) {
  return pack_f16x2(a, b);
}

// the lane's 10 elements of a row buffer as fp32 (chunk first, then pair)
template <typename T>
__device__ __forceinline__ void widen(const u32x4 c, uint32_t p, float (&v)[kPairElems]) {
  float c8[8];
  unpack<T>(c, c8);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = c8[e];
  unpack2<T>(p, v + 8);
}

// x and dout of one row; a row past the end sees empty buffers (reads 0,
// moves nothing)
template <typename T>
__device__ __forceinline__ void load_row(PairBatch& b, int64_t row, int64_t rows, const T* x,
                                         const T* dy, int n, int coff, int poff) {
  const bool ok = row < rows;
  const int64_t off = (ok ? row : 0) * static_cast<int64_t>(n);
  const uint32_t nb = ok ? static_cast<uint32_t>(n) * sizeof(T) : 0u;
  const rsrc_t xr = make_rsrc(x + off, nb);
  const rsrc_t gr = make_rsrc(dy + off, nb);
  b.xc = __builtin_amdgcn_raw_buffer_load_b128(xr, coff, 0, kStream);
  b.gc = __builtin_amdgcn_raw_buffer_load_b128(gr, coff, 0, kStream);
  b.xp = __builtin_amdgcn_raw_buffer_load_b32(xr, poff, 0, kStream);
  b.gp = __builtin_amdgcn_raw_buffer_load_b32(gr, poff, 0, kStream);
}

// the row's statistics through scalar loads (uniform over the workgroup;
// read-only for the whole kernel, which the constant address space asserts)
__device__ __forceinline__ void load_row_stats(PairBatch& b, int64_t row, int64_t rows,
                                               const float* mean, const float* rstd) {
  using cfloat = const __attribute__((address_space(4))) float;
  const bool ok = row < rows;
  b.rs = ok ? ((cfloat*)rstd)[row] : 0.0f;
  b.mu = ok ? ((cfloat*)mean)[row] : 0.0f;
}

}  // namespace

template <typename T, int PF>
__global__ void __launch_bounds__(512)
ln_gelu_bwd_pair(const T* dy, const T* x, const T* gamma, const T* beta, const float* mean,
                 const float* rstd, T* dx, float* part, int64_t part_stride, int64_t rows,
                 int n) {
  constexpr int E = kPairElems;
  __shared__ float red[4][16];  // [parity][sum] lines, one slot per wave
  const int t = threadIdx.x;
  const int nthr = blockDim.x;
  const int W = nthr >> 6;
  const int wave = wave_id();
  const int lane = t & 63;
  const float inv_n = 1.0f / static_cast<float>(n);
  const uint32_t rbytes = static_cast<uint32_t>(n) * sizeof(T);
  const int coff = t * 16;                                           // chunk t
  const int poff = (8 * nthr + 2 * t) * static_cast<int>(sizeof(T));  // pair t

  // gamma (1 where there is none) and beta (0), widened once
  float wv[E], bv[E];
  {
    const rsrc_t wr = make_rsrc(gamma, gamma != nullptr ? rbytes : 0u);
    const rsrc_t br = make_rsrc(beta, beta != nullptr ? rbytes : 0u);
    widen<T>(__builtin_amdgcn_raw_buffer_load_b128(wr, coff, 0, 0),
             __builtin_amdgcn_raw_buffer_load_b32(wr, poff, 0, 0), wv);
    widen<T>(__builtin_amdgcn_raw_buffer_load_b128(br, coff, 0, 0),
             __builtin_amdgcn_raw_buffer_load_b32(br, poff, 0, 0), bv);
    if (gamma == nullptr) {
#pragma unroll
      for (int e = 0; e < E; ++e) wv[e] = 1.0f;
    }
  }
  float acc1[E], acc2[E];  // column partials: dgamma (dy xhat) and dbeta (dy)
#pragma unroll
  for (int e = 0; e < E; ++e) {
    acc1[e] = 0.0f;
    acc2[e] = 0.0f;
  }

  // rows dealt out round robin (workgroup b: rows b, b + P, ...); PF rows
  // loaded ahead of the one being reduced, PF + 1 buffers used in turn
  const int64_t step = gridDim.x;
  int64_t base = blockIdx.x;
  PairBatch buf[PF + 1];
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    load_row<T>(buf[i], base + i * step, rows, x, dy, n, coff, poff);
    load_row_stats(buf[i], base + i * step, rows, mean, rstd);
  }
  int parity = 0;
  while (true) {
#pragma unroll
    for (int i = 0; i <= PF; ++i) {
      if (base >= rows) goto done;
      PairBatch& b = buf[i];
      PairBatch& ahead = buf[(i + PF) % (PF + 1)];
      const int64_t abase = base + PF * step;
      load_row<T>(ahead, abase, rows, x, dy, n, coff, poff);

      // first pass: dy = dout gelu'(pre-activation), g = dy gamma, kept for
      // the second pass with xhat; the row's two sums; the column partials.
      // (A row past the end is only ever loaded ahead, never processed.)
      float xv[E], dv[E], gdd[E], gxh[E];
      widen<T>(b.xc, b.xp, xv);
      widen<T>(b.gc, b.gp, dv);
      float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float xh = (xv[e] - b.mu) * b.rs;
        const float dd = dv[e] * gelu_tanh_grad(fmaf(xh, wv[e], bv[e]));
        const float gg = dd * wv[e];
        gdd[e] = gg;
        gxh[e] = xh;
        s1 += gg;
        s2 = fmaf(gg, xh, s2);
        acc2[e] += dd;
        acc1[e] = fmaf(dd, xh, acc1[e]);
      }
      s1 = wave_sum(s1);
      s2 = wave_sum(s2);
      if (W > 1) {
        // LDS lines double-buffered by row parity: one barrier per row
        float(*rp)[16] = red + 2 * parity;
        if (lane == 0) {
          rp[0][wave] = s1;
          rp[1][wave] = s2;
        }
        __syncthreads();
        s1 = slot_sum16(rp[0], 0, W);
        s2 = slot_sum16(rp[1], 0, W);
        parity ^= 1;
      }
      // the statistics of the row loaded ahead, once this row's sums are
      // complete (scalar loads share a wait counter with LDS; the asm takes
      // the finished sum and keeps memory operations from crossing it)
      asm volatile("" ::"s"(s1) : "memory");
      load_row_stats(ahead, abase, rows, mean, rstd);

      // second pass: dx = r (g - mean(g) - xhat mean(g xhat))
      const float k1 = -b.rs * (s1 * inv_n), k2 = -b.rs * (s2 * inv_n);
      float o[E];
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = fmaf(b.rs, gdd[e], fmaf(gxh[e], k2, k1));
      const bool ok = base < rows;
      const rsrc_t dr = make_rsrc(dx + (ok ? base : 0) * static_cast<int64_t>(n), ok ? rbytes : 0u);
      float o8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o8[e] = o[e];
      __builtin_amdgcn_raw_buffer_store_b128(pack<T>(o8), dr, coff, 0, kNormStore);
      __builtin_amdgcn_raw_buffer_store_b32(pack2<T>(o[8], o[9]), dr, poff, 0, kNormStore);
      base += step;
    }
  }
done:
  // this workgroup's fp32 partial rows: its columns' 10 values in each
  if (part != nullptr) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const uint32_t pbytes = static_cast<uint32_t>(n) * 4u;
    const rsrc_t p1 = make_rsrc(part + static_cast<int64_t>(blockIdx.x) * n, pbytes);
    const rsrc_t p2 = make_rsrc(part + part_stride + static_cast<int64_t>(blockIdx.x) * n, pbytes);
    const int c4 = t * 32;                     // the chunk's 8 columns as fp32
    const int p4 = (8 * nthr + 2 * t) * 4;     // the pair's 2 columns
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 v1, v2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v1[i] = __float_as_uint(acc1[4 * h + i]);
        v2[i] = __float_as_uint(acc2[4 * h + i]);
      }
      __builtin_amdgcn_raw_buffer_store_b128(v1, p1, c4 + 16 * h, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(v2, p2, c4 + 16 * h, 0, 0);
    }
    const u32x2 q1 = {__float_as_uint(acc1[8]), __float_as_uint(acc1[9])};
    const u32x2 q2 = {__float_as_uint(acc2[8]), __float_as_uint(acc2[9])};
    __builtin_amdgcn_raw_buffer_store_b64(q1, p1, p4, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b64(q2, p2, p4, 0, 0);
  }
}

bool ln_gelu_pair_fits(int dt, int64_t n, bool aligned) {
  return dt != 0 && aligned && n % 640 == 0 && (n / 640) % 4 == 0 && n / 640 <= 8;
}

hipError_t launch_ln_gelu_bwd_pair(int dt, int P, const void* dout, const void* x,
                                   const void* gamma, const void* beta, const float* mean,
                                   const float* rstd, void* dx, float* part, int64_t rows, int n,
                                   hipStream_t st) {
  if (!ln_gelu_pair_fits(dt, n, true) || P < 1) return hipErrorInvalidValue;
  const int W = n / 640;
  const int64_t part_stride = static_cast<int64_t>(P) * n;
  return by_dtype(dt, [&](auto tag) -> hipError_t {
    using T = decltype(tag);
    if constexpr (Vec<T>::N != 8) {
      return hipErrorInvalidValue;
    } else {
      hipLaunchKernelGGL((ln_gelu_bwd_pair<T, 3>), dim3(static_cast<unsigned>(P)), dim3(64 * W), 0,
                         st, static_cast<const T*>(dout), static_cast<const T*>(x),
                         static_cast<const T*>(gamma), static_cast<const T*>(beta), mean, rstd,
                         static_cast<T*>(dx), part, part_stride, rows, n);
      return hipGetLastError();
    }
  });
}

}  // namespace nr
