// nr_device.hpp -- device-side building blocks shared by the norm and RoPE
// kernels: 16-byte chunk I/O, bf16 <-> fp32 conversion and wave64 / workgroup
// reductions for gfx950 (CDNA4).
//
// Data model: a row (norms) or a token (RoPE) is cut into 16-byte chunks,
// 8 bf16 or fp16, or 4 fp32 elements each.  Lane t of a row group owns chunks
// t, t + 64W, t + 128W, ... so that every wave-wide load instruction touches
// 1 KiB of contiguous memory (fully coalesced global_load_dwordx4).  Chunks
// are kept in VGPRs as raw 32-bit words and widened to fp32 where used; every
// result is rounded to the storage type exactly once, when it is stored.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nr {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// bfloat16 storage tag: the top 16 bits of an IEEE single.
struct bf16 {
  uint16_t bits;
};
// IEEE binary16 storage tag.
struct f16 {
  uint16_t bits;
};

template <typename T> struct Vec;
template <> struct Vec<float> { static constexpr int N = 4; };
template <> struct Vec<bf16> { static constexpr int N = 8; };
template <> struct Vec<f16> { static constexpr int N = 8; };

// Calls f(T{}) with T the storage type of a dtype code (0 fp32, 1 bf16,
// 2 fp16): one place maps the C ABI's dtype onto kernel instantiations.
template <typename F>
__host__ hipError_t by_dtype(int dt, F&& f) {
  switch (dt) {
    case 0: return f(float{});
    case 1: return f(bf16{});
    case 2: return f(f16{});
  }
  return hipErrorInvalidValue;
}

// ---- conversions ---------------------------------------------------------

// fp32 pair -> packed bf16 pair, round to nearest even
// (gfx950 has a native instruction for this: v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// fp32 pair -> packed binary16 pair, round to nearest even
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}

// ---- 16-byte chunk <-> fp32 --------------------------------------------

template <typename T>
__device__ __forceinline__ void unpack(const u32x4 c, float (&v)[Vec<T>::N]);
template <>
__device__ __forceinline__ void unpack<float>(const u32x4 c, float (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(c[i]);
}
template <>
__device__ __forceinline__ void unpack<bf16>(const u32x4 c, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(c[i] << 16);
    v[2 * i + 1] = __uint_as_float(c[i] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void unpack<f16>(const u32x4 c, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // through a named word: hipcc (ROCm 7.2) lowers a bit_cast of the
    // subscript c[i] itself as a cast of c[0]
    const uint32_t word = c[i];
    const f32x2 f = __builtin_convertvector(__builtin_bit_cast(f16x2, word), f32x2);
    v[2 * i] = f[0];
    v[2 * i + 1] = f[1];
  }
}

template <typename T>
__device__ __forceinline__ u32x4 pack(const float (&v)[Vec<T>::N]);
template <>
__device__ __forceinline__ u32x4 pack<float>(const float (&v)[4]) {
  u32x4 c;
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = __float_as_uint(v[i]);
  return c;
}
template <>
__device__ __forceinline__ u32x4 pack<bf16>(const float (&v)[8]) {
  u32x4 c;
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  return c;
}
template <>
__device__ __forceinline__ u32x4 pack<f16>(const float (&v)[8]) {
  u32x4 c;
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = pack_f16x2(v[2 * i], v[2 * i + 1]);
  return c;
}

// ---- buffer resources --------------------------------------------------
//
// Rows and tokens are read and written through buffer resources: a
// wave-uniform descriptor (base address, size in bytes) held in SGPRs plus a
// 32-bit per-lane byte offset.  The hardware range-checks every access
// against the size: a load past the end returns 0 and a store past the end
// is dropped.  So lanes that own no chunk of a short row, or a whole row
// group past the last row, need no branch, and no lane carries a 64-bit
// pointer.  Word 3 (0x00020000) is the gfx9-family setting for raw
// (unswizzled, stride 0) 32-bit buffer access.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Cache policy of the streaming row traffic (x, y, dy, dx, RoPE data): the
// buffer instructions' aux bits; 2 sets "nt" (non-temporal) on gfx950, which
// measured 4-20% faster than the default policy on every kernel here (the
// data is touched once per kernel).  Weights, statistics and tables, which
// are re-read, keep the default (0).
#ifndef NR_STREAM_AUX
#define NR_STREAM_AUX 2
#endif
constexpr int kStream = NR_STREAM_AUX;
// Stores of the in-place RoPE kernel (and of the ceiling copy) add sc1
// (bit 4, system scope) to nt: a plain copy ran about 2% faster this way
// (6.66 against 6.53 TB/s on MI355X) and RoPE about 1%; sc0 or sc1 on the
// loads gained nothing further.  The norm kernels keep nt on their stores:
// with sc1 their backward and the 3840-row Gemma step measured 1-2% slower.
#ifndef NR_STREAM_STORE_AUX
#define NR_STREAM_STORE_AUX 18
#endif
constexpr int kStreamStore = NR_STREAM_STORE_AUX;
// Stores of the norm kernels' outputs (y, dx).
#ifndef NR_NORM_STORE_AUX
#define NR_NORM_STORE_AUX NR_STREAM_AUX
#endif
constexpr int kNormStore = NR_NORM_STORE_AUX;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// Chunk c (elements [cE, cE + E)) of a buffer.  VEC: one 128-bit access (the
// buffer starts 16-byte aligned and holds whole chunks).  Otherwise element
// by element, each access naturally aligned and range-checked on its own;
// that path serves odd shapes and alignments, not speed.
template <typename T, bool VEC, int AUX = 0>
__device__ __forceinline__ u32x4 ld_chunk(rsrc_t r, int c) {
  if constexpr (VEC) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, c * 16, 0, AUX);
  } else if constexpr (Vec<T>::N == 8) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, (c * 8 + 2 * i) * 2, 0, 0);
      const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(r, (c * 8 + 2 * i + 1) * 2, 0, 0);
      v[i] = lo | (hi << 16);
    }
    return v;
  } else {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b32(r, (c * 4 + i) * 4, 0, 0);
    return v;
  }
}

template <typename T, bool VEC, int AUX = 0>
__device__ __forceinline__ void st_chunk(rsrc_t r, int c, const u32x4 v) {
  if constexpr (VEC) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, c * 16, 0, AUX);
  } else if constexpr (Vec<T>::N == 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(v[i] & 0xffffu), r,
                                            (c * 8 + 2 * i) * 2, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(v[i] >> 16), r,
                                            (c * 8 + 2 * i + 1) * 2, 0, 0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) __builtin_amdgcn_raw_buffer_store_b32(v[i], r, (c * 4 + i) * 4, 0, 0);
  }
}

// single fp32 / element access through a buffer
__device__ __forceinline__ float ld_f32(rsrc_t r, int byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}
__device__ __forceinline__ void st_f32(rsrc_t r, int byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, byte_off, 0, 0);
}
template <typename T> __device__ __forceinline__ float ld_elem(rsrc_t r, int byte_off);
template <> __device__ __forceinline__ float ld_elem<float>(rsrc_t r, int byte_off) {
  return ld_f32(r, byte_off);
}
template <> __device__ __forceinline__ float ld_elem<bf16>(rsrc_t r, int byte_off) {
  return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, byte_off, 0, 0)) << 16);
}
template <> __device__ __forceinline__ float ld_elem<f16>(rsrc_t r, int byte_off) {
  const uint16_t h = static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(r, byte_off, 0, 0));
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}
template <typename T> __device__ __forceinline__ void st_elem(rsrc_t r, int byte_off, float v);
template <> __device__ __forceinline__ void st_elem<float>(rsrc_t r, int byte_off, float v) {
  st_f32(r, byte_off, v);
}
template <> __device__ __forceinline__ void st_elem<bf16>(rsrc_t r, int byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(pack_bf16x2(v, 0.0f) & 0xffffu), r,
                                        byte_off, 0, 0);
}
template <> __device__ __forceinline__ void st_elem<f16>(rsrc_t r, int byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(pack_f16x2(v, 0.0f) & 0xffffu), r,
                                        byte_off, 0, 0);
}

// ---- interleaved RoPE helpers ------------------------------------------

// PP consecutive fp32 entries starting at entry e0 of a table row buffer
template <int PP>
__device__ __forceinline__ void load_tab(rsrc_t r, int e0, float (&v)[PP]) {
  if constexpr (PP == 4) {
    const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, e0 * 4, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(t[i]);
  } else if constexpr (PP == 2) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, e0 * 4, 0, 0);
    v[0] = __uint_as_float(t[0]);
    v[1] = __uint_as_float(t[1]);
  } else {
#pragma unroll
    for (int i = 0; i < PP; ++i) v[i] = ld_f32(r, (e0 + i) * 4);
  }
}

// Rotate the pairs (v[2p], v[2p+1]) = (real, imaginary) of a chunk by their
// angles: a' = a c - b (sign s), b' = a (sign s) + b c; sign = -1 is the
// inverse rotation.
template <int PP>
__device__ __forceinline__ void rotate_pairs(float* v, const float (&c)[PP], const float (&s)[PP],
                                             float sign) {
#pragma unroll
  for (int p = 0; p < PP; ++p) {
    const float sn = sign * s[p];
    const float a = v[2 * p], b = v[2 * p + 1];
    v[2 * p] = fmaf(a, c[p], -(b * sn));
    v[2 * p + 1] = fmaf(a, sn, b * c[p]);
  }
}

// ---- tanh-approximated GeLU --------------------------------------------
//
// gelu(v) = v/2 (1 + tanh(u)), u = c (v + 0.044715 v^3), c = sqrt(2/pi).
// Since 1 + tanh(u) = 2 / (1 + exp(-2u)), it is evaluated as
// v / (1 + exp(-2u)), which does not cancel for v << 0 and saturates to 0
// or v.  The derivative, with s = 1/(1 + exp(-2u)) and 1 - s = exp(-2u) s:
//   gelu'(v) = s + 2 v s (1 - s) c (1 + 3 * 0.044715 v^2).
//
// The activation runs once per element of an HBM-bound row kernel, so its
// ALU cost is what decides whether the fused kernel keeps up with memory:
// exp(-2u) is one hardware base-2 exponential of v (k0 + k1 v^2) (the
// constants fold -2 c log2(e) in), and the divisions are hardware
// reciprocals (about 1 ulp each).  Rounding the exponent's argument costs
// a relative error of |arg| * 2^-24 * ln 2 in exp(-2u), a few 1e-6 at most
// where the sigmoid is not saturated: well inside an fp32 tolerance of
// 1e-5 and far inside one bf16 ulp.
constexpr double kGeluCd = 0.79788456080286535588;  // sqrt(2/pi)
constexpr double kLog2e = 1.44269504088896340736;
constexpr float kGeluK0 = static_cast<float>(-2.0 * kGeluCd * kLog2e);
constexpr float kGeluK1 = static_cast<float>(-2.0 * kGeluCd * kLog2e * 0.044715);
constexpr float kGeluT0 = static_cast<float>(2.0 * kGeluCd);           // 2c
constexpr float kGeluT1 = static_cast<float>(2.0 * kGeluCd * 3.0 * 0.044715);  // 6ac

// exp(-2u) for the activation's argument v, u = c (v + a v^3) (one v_exp_f32
// of the base-2 exponent).  It may overflow to +inf for v << 0; both users
// take that limit correctly, so no cap (and no v_min) is needed.
__device__ __forceinline__ float gelu_exp(float v) {
  return __builtin_amdgcn_exp2f(v * fmaf(kGeluK1, v * v, kGeluK0));
}

__device__ __forceinline__ float gelu_tanh(float v) {
  // exp = inf gives v * 0 = -0, the limit for v -> -inf
  return v * __builtin_amdgcn_rcpf(1.0f + gelu_exp(v));
}

__device__ __forceinline__ float gelu_tanh_grad(float v) {
  // s + t s (1 - s) with 1 - s formed by subtraction: exact for s >= 1/2,
  // and for v -> -inf (exp = inf, s = 0) the product is t * 0 * 1 = 0
  // rather than inf * 0
  const float e = gelu_exp(v);
  const float s = __builtin_amdgcn_rcpf(1.0f + e);
  const float t = v * fmaf(kGeluT1, v * v, kGeluT0);  // 2 c v (1 + 3a v^2)
  return fmaf(t * s, 1.0f - s, s);
}

// Epilogues of the fused row kernels
constexpr int kEpiNone = 0;
constexpr int kEpiRope = 1;  // RMSNorm output rotated as interleaved RoPE pairs
constexpr int kEpiGelu = 2;  // LayerNorm output through the tanh-approximated GeLU

// index of the calling wave within its workgroup, as a scalar (SGPR) value
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
}

// ---- reductions ----------------------------------------------------------

// lane i reads lane (pattern) of the same 16-lane DPP row
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wave; every lane gets the same bits.
// Within a 16-lane row: butterfly over quad_perm [1,0,3,2], quad_perm
// [2,3,0,1], row_half_mirror and row_mirror (each lane adds a partner that
// holds a disjoint partial sum, so all lanes of the row end up equal).
// Across rows: gfx950's v_permlane16_swap / v_permlane32_swap exchange
// whole rows in VALU, with no LDS round trip.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  {
    const uint32_t u = __float_as_uint(v);
    auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  {
    const uint32_t u = __float_as_uint(v);
    auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  return v;
}

// Sum over the S consecutive lanes (S a power of two, 4..32) that hold one
// row; lanes that hold disjoint partial sums are added pairwise.
template <int S>
__device__ __forceinline__ float lane_group_sum(float v) {
  v += dpp<0xB1>(v);  // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);  // quad_perm [2,3,0,1]
  if constexpr (S >= 8) v += dpp<0x141>(v);  // row_half_mirror: the other quad
  if constexpr (S >= 16) v += dpp<0x140>(v);  // row_mirror: the other half-row
  if constexpr (S >= 32) {
    // rows 0 <-> 1 and 2 <-> 3 of the wave
    const uint32_t u = __float_as_uint(v);
    auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  return v;
}

// Sum of the slots [lo, hi) of a 16-float LDS line that the waves of a
// workgroup have filled (one slot per wave), returned as a uniform value.
// One LDS read per lane, whatever the number of waves: lane i of each
// 16-lane row reads slot i, slots outside [lo, hi) (another row group's, or
// never written) are replaced by 0, and the row's first four butterfly steps
// of wave_sum add the 16 in a fixed tree; every wave that asks gets the same
// bits.
__device__ __forceinline__ float slot_sum16(const float* line, int lo, int hi) {
  const int i = threadIdx.x & 15;
  float v = line[i];
  v = (i >= lo && i < hi) ? v : 0.0f;
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// Sum of v over the W waves of a row group (W == 1: a pure wave reduction).
// red: LDS scratch of at least blockDim/64 floats, used once per call site;
// wave sums meet there and are added in wave order.
__device__ __forceinline__ float group_sum(float v, int W, int wave, int g, float* red) {
  v = wave_sum(v);
  if (W == 1) return v;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float s = 0.0f;
  for (int i = 0; i < W; ++i) s += red[g * W + i];
  return s;
}

// Make the compiler treat these registers as freshly written, so values it
// derived from them earlier (widened fp32 copies, products) are recomputed
// rather than kept alive across a reduction.  Only the packed 16-byte chunks
// stay resident, which halves the VGPRs a bf16 row needs.
template <int N>
__device__ __forceinline__ void reload_barrier(u32x4 (&a)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(a[i]));
}

}  // namespace nr
