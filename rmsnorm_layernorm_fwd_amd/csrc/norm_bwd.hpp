// norm_bwd.hpp -- RMSNorm / LayerNorm backward for gfx950 (stage 1 of the
// deterministic column reduction that finishes dW, dgamma and dbeta).
//
// The backward reads each row's cached statistic (inverse root; LayerNorm
// also the mean) instead of recomputing it (Helios 性能优化全解析, 内核一
// FlashNorm: the forward stores each row's inverse statistic and the backward
// uses it directly).  x and dy are each read once, dx written once.
//
// Mapping (stage 1): a workgroup of W waves works on D rows at a time, all W
// waves on every row, so a lane owns the same columns throughout and adds
// dy * xhat (and dy) for them into fp32 registers: the column gradients need
// no atomics and no extra pass over the rows.  Batches are dealt out
// round-robin -- workgroup b takes rows b*D.., then b*D + P*D.., ... -- so at
// any moment the whole grid streams one contiguous window of the tensor,
// which keeps DRAM pages open (contiguous per-workgroup ranges would spread
// P concurrent streams over the whole tensor).  The next batch is loaded
// before the current one is reduced (two register buffers used in turn, so
// no copy forces a wait on the prefetch), which keeps loads in flight across
// the reduction's barrier.  A batch's D row sums are wave-reduced together
// and meet in one LDS round with one barrier (LDS double-buffered by batch
// parity, so there is no second barrier).  At the end each workgroup writes
// its fp32 partial row; stage 2 adds the partial rows column by column in
// workgroup order.  Every summation order is fixed by the shape, so the
// results are bitwise reproducible run to run.
#pragma once

#include "nr_device.hpp"
#include "nr_internal.hpp"

namespace nr {

//   RMS: xhat = x r, g = dy w', c = sum(g xhat)/n, dx = r (g - xhat c),
//        partial dW += dy xhat
//   LN:  xhat = (x - mu) r, g = dy gamma, a = sum(g)/n, bb = sum(g xhat)/n,
//        dx = r (g - a - xhat bb), partial dgamma += dy xhat, dbeta += dy
// part: [2][P][n] fp32 (second matrix, at part + part_stride, for dbeta);
// null when no column gradient is wanted.
// D rows of x and dy as loaded (packed), their statistics and, for the fused
// RMSNorm + RoPE backward, the cos/sin of TS table slots per row: TS = K, one
// per chunk, or TS = 1 when all of a lane's chunks sit at the same offset in
// their heads (the row's lane stride a multiple of the head size), which
// halves the table registers of two chunks per lane; TS = 0 without RoPE.
template <typename T, int K, int D, int TS>
struct RowBatch {
  u32x4 x[D * K], g[D * K];
  float rs[D], mu[D];
  float tc[D * TS][Vec<T>::N / 2], ts[D * TS][Vec<T>::N / 2];
};

// A batch's row statistics as scalar loads (into SGPRs: each is uniform over
// the workgroup).  They are read-only for the kernel's whole run, which is
// what the constant address space asserts.  Rows past the end take 0 and load
// nothing.
template <typename T, int K, int D, bool LN, int TS>
__device__ __forceinline__ void load_stats(RowBatch<T, K, D, TS>& b, int64_t base, int64_t rows,
                                           const float* mean, const float* rstat) {
  using cfloat = const __attribute__((address_space(4))) float;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const int64_t row = base + d;
    const bool okr = row < rows;
    b.rs[d] = okr ? ((cfloat*)rstat)[row] : 0.0f;
    b.mu[d] = (LN && okr) ? ((cfloat*)mean)[row] : 0.0f;
  }
}

// SSTAT: the statistics are left to load_stats, issued later.
template <typename T, int K, int D, bool VEC, bool LN, bool ROPE, int TS, bool SSTAT>
__device__ __forceinline__ void load_batch(RowBatch<T, K, D, TS>& b, int64_t base,
                                           int64_t rows, const T* x, const T* dy,
                                           const float* mean, const float* rstat, int n, int t,
                                           int nthr, const RopeArgs& ra) {
  constexpr int E = Vec<T>::N;
  const uint32_t rbytes = static_cast<uint32_t>(n) * sizeof(T);
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const int64_t row = base + d;
    const bool okr = row < rows;
    const int64_t off = (okr ? row : 0) * static_cast<int64_t>(n);
    const uint32_t nb = okr ? rbytes : 0u;  // rows past the end read as 0, move no data
    const rsrc_t xr = make_rsrc(x + off, nb);
    const rsrc_t gr = make_rsrc(dy + off, nb);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      b.x[d * K + k] = ld_chunk<T, VEC, kStream>(xr, t + k * nthr);
      b.g[d * K + k] = ld_chunk<T, VEC, kStream>(gr, t + k * nthr);
    }
    if constexpr (!SSTAT) {
      b.rs[d] = okr ? rstat[row] : 0.0f;
      b.mu[d] = (LN && okr) ? mean[row] : 0.0f;
    }
    if constexpr (ROPE) {
      // the token's table rows; this lane's chunks sit at fixed offsets in
      // their heads (see the forward)
      constexpr int PP = E / 2;
      const int half = ra.head_dim >> 1;
      const int64_t tok = (okr ? row : 0) / ra.rows_per_token;
      const uint32_t tb = okr ? static_cast<uint32_t>(half) * 4u : 0u;
      const rsrc_t cr = make_rsrc(ra.cos_tab + tok * half, tb);
      const rsrc_t sr = make_rsrc(ra.sin_tab + tok * half, tb);
      int hoff = (t * E) % ra.head_dim;
      const int hstep = (nthr * E) % ra.head_dim;
#pragma unroll
      for (int k = 0; k < TS; ++k) {
        if constexpr (VEC) {
          load_tab<PP>(cr, hoff >> 1, b.tc[d * TS + k]);
          load_tab<PP>(sr, hoff >> 1, b.ts[d * TS + k]);
        } else {
#pragma unroll
          for (int p = 0; p < PP; ++p) {
            const int ho = (hoff + 2 * p) % ra.head_dim;
            b.tc[d * TS + k][p] = ld_f32(cr, (ho >> 1) * 4);
            b.ts[d * TS + k][p] = ld_f32(sr, (ho >> 1) * 4);
          }
        }
        hoff += hstep;
        if (hoff >= ra.head_dim) hoff -= ra.head_dim;
      }
    }
  }
}

// dy of chunk i as fp32: the loaded values, rotated back by the token's
// angles when the upstream gradient is that of a RoPE output
template <typename T, int K, int D, bool ROPE, int TS>
__device__ __forceinline__ void dy_chunk(const RowBatch<T, K, D, TS>& b, int i,
                                         float (&dv)[Vec<T>::N]) {
  unpack<T>(b.g[i], dv);
  if constexpr (ROPE) {
    const int slot = TS == K ? i : i / K;  // chunk i = d K + k of row d
    rotate_pairs<Vec<T>::N / 2>(dv, b.tc[slot], b.ts[slot], -1.0f);
  }
}

// EPI == kEpiGelu (LayerNorm): the upstream gradient is that of
// gelu(xhat gamma + beta); the pre-activation is recomputed from the cached
// statistics and dy = dout * gelu'(pre-activation).
// late(): with SSTAT, issues the scalar statistics loads of a batch loaded
// ahead, once this batch's sums are complete.  Scalar loads complete out of
// order, so every wait for one (and for an LDS access: they share a counter)
// waits for all; issued here, after the sums' LDS read has been waited for,
// they have the rest of this batch and the next batch's first pass before
// the next such wait.
template <typename T, int K, int D, bool VEC, bool LN, bool ROPE, int EPI, int TS, bool SSTAT,
          bool LACC, typename F>
__device__ __forceinline__ void process_batch(RowBatch<T, K, D, TS>& b, int64_t base,
                                              int64_t rows, T* dx, int n, int t, int nthr, int W,
                                              int wave, int lane, float inv_n,
                                              const float (&wv)[K][Vec<T>::N],
                                              const float (&bv)[K][Vec<T>::N],
                                              const u32x4 (&wpk)[K], const u32x4 (&bpk)[K],
                                              float w_add, float (&acc1)[K][Vec<T>::N],
                                              float (&acc2)[K][Vec<T>::N],
                                              float4* lacc, float (*red)[16], int& parity,
                                              F&& late) {
  constexpr int E = Vec<T>::N;
  constexpr int NS = LN ? 2 : 1;  // row sums per row
  // per-lane partial row sums, and the column partials.  Elements past n
  // (and rows past the end) were read as 0, so their dy is 0 and every
  // term they contribute is 0 times a finite value: no mask is needed,
  // LayerNorm's centred xhat = -mean * rstd there included.
  float s[NS * D];
  // GeLU: dy * gamma with dy = dout * gelu'(pre-activation), kept for the
  // second pass (the activation's derivative is the costliest arithmetic
  // here).  With one chunk per lane xhat is kept too.  With more (LEAN) it
  // is recomputed from x in the second pass, and gamma and beta stay packed
  // and are widened per batch (behind a register barrier, so the compiler
  // cannot hoist the widened copies out of the row loop): this keeps the
  // 1024-thread kernel within its 128 VGPRs, where it spilled before.
  constexpr int GD = EPI == kEpiGelu ? D * K : 0;
  constexpr bool LEAN = EPI == kEpiGelu && K > 1;
  // LACC (RMSNorm rows of 16385..32768 elements): the weight stays packed as
  // for LEAN, and dW is accumulated in LDS, in the second pass
  constexpr bool PACKW = LEAN || LACC;
  float gdd[GD > 0 ? GD : 1][E], gxh[(GD > 0 && !LEAN) ? GD : 1][E];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      float xv[E], dv[E], wl[E], bl[E];
      unpack<T>(b.x[d * K + k], xv);
      dy_chunk<T, K, D, ROPE, TS>(b, d * K + k, dv);
      if constexpr (PACKW) {
        u32x4 wq[1] = {wpk[k]};
        reload_barrier<1>(wq);
        unpack<T>(wq[0], wl);
      }
      if constexpr (LEAN) {
        u32x4 bq[1] = {bpk[k]};
        reload_barrier<1>(bq);
        unpack<T>(bq[0], bl);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float xh = (xv[e] - b.mu[d]) * b.rs[d];
        const float wk = PACKW ? wl[e] + w_add : wv[k][e];
        float dd = dv[e];
        if constexpr (EPI == kEpiGelu)
          dd *= gelu_tanh_grad(fmaf(xh, wk, LEAN ? bl[e] : bv[k][e]));
        const float gg = dd * wk;
        if constexpr (EPI == kEpiGelu) {
          gdd[d * K + k][e] = gg;
          if constexpr (!LEAN) gxh[d * K + k][e] = xh;
        }
        if constexpr (LN) {
          s1 += gg;
          s2 = fmaf(gg, xh, s2);
          acc2[k][e] += dd;
        } else {
          s1 = fmaf(gg, xh, s1);
        }
        if constexpr (!LACC) acc1[k][e] = fmaf(dd, xh, acc1[k][e]);
      }
    }
    s[NS * d] = s1;
    if constexpr (LN) s[NS * d + 1] = s2;
  }
  if constexpr (EPI != kEpiGelu) {
    reload_barrier<D * K>(b.x);
    reload_barrier<D * K>(b.g);
  }

  // reduce the batch's NS*D sums across the workgroup
#pragma unroll
  for (int i = 0; i < NS * D; ++i) s[i] = wave_sum(s[i]);
  if (W > 1) {
    float(*rp)[16] = red + parity * (NS * D);
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < NS * D; ++i) rp[i][wave] = s[i];
    }
    __syncthreads();
    // The GeLU backward, whose activation arithmetic already stands between
    // a batch's loads and its barrier, adds the W wave sums with one LDS read
    // and a 16-lane tree (15360 x 5120 bf16: 110.1 -> 102.9 us).  The others
    // keep the in-order loop over the slots: measured against the tree on
    // one MI355X, the RMSNorm and LayerNorm backward at 65536 x 5120 bf16
    // ran 3-6% slower with it (329.6 -> 338.9 and 325.0 -> 343.5 us) and the
    // forwards no faster.
#pragma unroll
    for (int i = 0; i < NS * D; ++i) {
      if constexpr (EPI == kEpiGelu) {
        s[i] = slot_sum16(rp[i], 0, W);
      } else {
        float tot = 0.0f;
        for (int q = 0; q < W; ++q) tot += rp[i][q];
        s[i] = tot;
      }
    }
    parity ^= 1;  // the other buffer next batch: no second barrier needed
  }
  if constexpr (SSTAT) {
    // the asm needs the finished sum, and memory operations cannot cross it
    asm volatile("" ::"s"(s[0]) : "memory");
    late();
  }

  const uint32_t rbytes = static_cast<uint32_t>(n) * sizeof(T);
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const int64_t row = base + d;
    const bool okr = row < rows;
    const rsrc_t dr = make_rsrc(dx + (okr ? row : 0) * static_cast<int64_t>(n), okr ? rbytes : 0u);
    const float c1 = s[NS * d] * inv_n;
    const float c2 = LN ? s[NS * d + 1] * inv_n : 0.0f;
    // LayerNorm: dx = r g - (r c1 + r c2 xhat), the bracket one fma per
    // element with the row constants folded in
    const float k1 = -b.rs[d] * c1, k2 = -b.rs[d] * c2;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      float xv[E], dv[E], o[E], wl[E], xhv[E];
      if constexpr (EPI != kEpiGelu || LEAN) unpack<T>(b.x[d * K + k], xv);
      if constexpr (EPI != kEpiGelu) dy_chunk<T, K, D, ROPE, TS>(b, d * K + k, dv);
      if constexpr (LACC) {
        u32x4 wq[1] = {wpk[k]};
        reload_barrier<1>(wq);
        unpack<T>(wq[0], wl);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float xh, gg;
        if constexpr (EPI == kEpiGelu) {
          gg = gdd[d * K + k][e];
          xh = LEAN ? (xv[e] - b.mu[d]) * b.rs[d] : gxh[d * K + k][e];
        } else {
          gg = dv[e] * (LACC ? wl[e] + w_add : wv[k][e]);
          xh = (xv[e] - b.mu[d]) * b.rs[d];
        }
        xhv[e] = xh;
        if constexpr (LN) {
          o[e] = fmaf(b.rs[d], gg, fmaf(xh, k2, k1));
        } else {
          o[e] = b.rs[d] * (gg - xh * c1);
        }
      }
      st_chunk<T, VEC, kNormStore>(dr, t + k * nthr, pack<T>(o));
      if constexpr (LACC) {
        // this lane's own slots (no other lane touches them): the same fma,
        // in the same row order, as the register accumulators would take
        float4* slot = lacc + (k * (E / 4)) * 1024 + t;
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
          float4 a = slot[q * 1024];
          a.x = fmaf(dv[4 * q + 0], xhv[4 * q + 0], a.x);
          a.y = fmaf(dv[4 * q + 1], xhv[4 * q + 1], a.y);
          a.z = fmaf(dv[4 * q + 2], xhv[4 * q + 2], a.z);
          a.w = fmaf(dv[4 * q + 3], xhv[4 * q + 3], a.w);
          slot[q * 1024] = a;
        }
      }
    }
  }
}

// LB: the largest workgroup the instantiation serves.  1024 (16 waves) caps
// a lane at 128 VGPRs; the deep-prefetch instantiations (PF 3, 4) take at
// most 10 waves, i.e. one workgroup per CU, which leaves up to 168.
// SHARED (RoPE, more than one chunk per lane): one set of table angles per
// row, valid when the lane stride of the row is a multiple of the head size.
// LACC (plain RMSNorm, aligned 16-bit rows, 4 chunks = 32 elements per lane,
// one row per batch, one batch ahead): the 32 fp32 dW accumulators of each
// lane live in 128 KiB of LDS, one workgroup per CU, where in registers they
// spilled; rows of 16385..32768 elements then take one pass instead of two.
template <typename T, int K, int D, int PF, bool VEC, bool LN, int EPI, int LB = 1024,
          bool SHARED = false, bool LACC = false>
__global__ void __launch_bounds__(LB)
norm_bwd_rows(const T* dy, const T* x, const T* w, const T* beta, const float* mean,
              const float* rstat, T* dx, float* part, int64_t part_stride, int64_t rows, int n,
              float w_add, RopeArgs ra) {
  constexpr bool ROPE = EPI == kEpiRope;
  constexpr int TS = ROPE ? (SHARED ? 1 : K) : 0;
  constexpr int E = Vec<T>::N;
  constexpr int NS = LN ? 2 : 1;
  __shared__ float red[2 * NS * D][16];
  const int t = threadIdx.x;
  const int nthr = blockDim.x;
  const int W = nthr >> 6;
  const int wave = wave_id();
  const int lane = t & 63;
  const float inv_n = 1.0f / static_cast<float>(n);
  const uint32_t rbytes = static_cast<uint32_t>(n) * sizeof(T);

  // the weight (1 where there is none), widened once; or, for the GeLU
  // backward with more than one chunk per lane, kept packed (ones packed
  // where there is no weight, the offset applied where it is widened)
  constexpr bool LEAN = EPI == kEpiGelu && K > 1;
  static_assert(!LACC || (!LN && EPI == kEpiNone && D == 1 && PF == 1 && K * E == 32 &&
                          LB == 1024 && VEC),
                "LDS accumulators: plain aligned RMSNorm, 32 elements a lane, one batch ahead");
  constexpr int LQ = K * E / 4;  // float4 accumulator slots per lane
  __shared__ float4 lacc[LACC ? LQ * 1024 : 1];
  float wv[K][E];
  u32x4 wpk[K];
  const float w_add_packed = (w != nullptr) ? w_add : 0.0f;
  {
    const rsrc_t wr = make_rsrc(w, w != nullptr ? rbytes : 0u);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      wpk[k] = ld_chunk<T, VEC>(wr, t + k * nthr);
      if constexpr (LEAN || LACC) {
        if (w == nullptr) {
          float one[E];
#pragma unroll
          for (int e = 0; e < E; ++e) one[e] = 1.0f;
          wpk[k] = pack<T>(one);
        }
      } else {
        unpack<T>(wpk[k], wv[k]);
#pragma unroll
        for (int e = 0; e < E; ++e) wv[k][e] = (w != nullptr) ? wv[k][e] + w_add : 1.0f;
      }
    }
  }

  // beta, only read by the GeLU epilogue: widened once, or (more than one
  // chunk per lane) kept packed and widened where used
  float bv[K][E];
  u32x4 bpk[K];
  {
    const rsrc_t br = make_rsrc(beta, (EPI == kEpiGelu && beta != nullptr) ? rbytes : 0u);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      bpk[k] = ld_chunk<T, VEC>(br, t + k * nthr);
      if constexpr (!LEAN) unpack<T>(bpk[k], bv[k]);
    }
  }

  float acc1[K][E], acc2[K][E];
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      acc1[k][e] = 0.0f;
      acc2[k][e] = 0.0f;
    }
  if constexpr (LACC) {
#pragma unroll
    for (int q = 0; q < LQ; ++q) lacc[q * 1024 + t] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }

  int parity = 0;
  const int64_t step = static_cast<int64_t>(gridDim.x) * D;
  int64_t base = static_cast<int64_t>(blockIdx.x) * D;
  // PF batches are loaded ahead of the one being reduced; PF + 1 register
  // buffers are used in turn (the loop is unrolled over them, so no register
  // copy ever waits on a load in flight).
  //
  // The row statistics of the LayerNorm (with or without GeLU) and RoPE
  // backward come in through scalar loads (SSTAT), which frees their VGPRs in
  // every buffer.  Measured on MI355X (bf16, rows of 5120): LayerNorm + GeLU
  // at 15360 rows 103 -> 94 us, RMSNorm + RoPE at 65536 rows 349 -> 324 us,
  // LayerNorm 85.4 -> 82.5 us at 15360 rows and level at 65536; the plain
  // RMSNorm backward ran about 1% slower with them and keeps vector loads.
  constexpr bool SSTAT = LN || ROPE;
  RowBatch<T, K, D, TS> buf[PF + 1];
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    load_batch<T, K, D, VEC, LN, ROPE, TS, SSTAT>(buf[i], base + i * step, rows, x, dy, mean, rstat,
                                                  n, t, nthr, ra);
    if constexpr (SSTAT) load_stats<T, K, D, LN, TS>(buf[i], base + i * step, rows, mean, rstat);
  }
  while (true) {
#pragma unroll
    for (int i = 0; i <= PF; ++i) {
      if (base >= rows) goto done;
      RowBatch<T, K, D, TS>& ahead = buf[(i + PF) % (PF + 1)];
      const int64_t abase = base + PF * step;
      load_batch<T, K, D, VEC, LN, ROPE, TS, SSTAT>(ahead, abase, rows, x, dy, mean, rstat, n, t,
                                                    nthr, ra);
      process_batch<T, K, D, VEC, LN, ROPE, EPI, TS, SSTAT, LACC>(
          buf[i], base, rows, dx, n, t, nthr, W, wave, lane, inv_n, wv, bv, wpk, bpk, w_add_packed,
          acc1, acc2, lacc, red, parity, [&] {
            if constexpr (SSTAT) load_stats<T, K, D, LN, TS>(ahead, abase, rows, mean, rstat);
          });
      base += step;
    }
  }
done:

  // this workgroup's fp32 partial row(s) of the column gradients
  if (part != nullptr) {
    const uint32_t pbytes = static_cast<uint32_t>(n) * 4u;
    const rsrc_t p1 = make_rsrc(part + static_cast<int64_t>(blockIdx.x) * n, pbytes);
    const rsrc_t p2 = make_rsrc(part + part_stride + static_cast<int64_t>(blockIdx.x) * n,
                                LN ? pbytes : 0u);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int c = t + k * nthr;
#pragma unroll
      for (int q = 0; q < E / 4; ++q) {
        if constexpr (LACC) {
          const float4 a = lacc[(k * (E / 4) + q) * 1024 + t];
          acc1[k][4 * q + 0] = a.x;
          acc1[k][4 * q + 1] = a.y;
          acc1[k][4 * q + 2] = a.z;
          acc1[k][4 * q + 3] = a.w;
        }
        if constexpr (VEC) {
          // whole 16-byte groups of 4 columns (n is a multiple of 4 here)
          u32x4 v1, v2;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v1[i] = __float_as_uint(acc1[k][4 * q + i]);
            v2[i] = __float_as_uint(acc2[k][4 * q + i]);
          }
          __builtin_amdgcn_raw_buffer_store_b128(v1, p1, (c * E + 4 * q) * 4, 0, 0);
          if constexpr (LN) __builtin_amdgcn_raw_buffer_store_b128(v2, p2, (c * E + 4 * q) * 4, 0, 0);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            st_f32(p1, (c * E + 4 * q + i) * 4, acc1[k][4 * q + i]);
            if constexpr (LN) st_f32(p2, (c * E + 4 * q + i) * 4, acc2[k][4 * q + i]);
          }
        }
      }
    }
  }
}


template <typename T, int K, int D, bool A, bool LN, int EP>
hipError_t launch_bwd_kd(const BwdPlan& pl, const void* dy, const void* x, const void* w,
                         const void* beta, const float* mean, const float* rstat, void* dx,
                         float* part, int64_t rows, int n, float w_add, const RopeArgs& ra,
                         hipStream_t st) {
  const int64_t part_stride = static_cast<int64_t>(pl.P) * n;
  auto kern = pl.PF == 2 ? norm_bwd_rows<T, K, D, 2, A, LN, EP> : norm_bwd_rows<T, K, D, 1, A, LN, EP>;
  if constexpr (K == 1 && D <= 2) {
    if (pl.PF >= 3) {
      if (pl.W > 10) return hipErrorInvalidValue;
      kern = pl.PF == 3 ? norm_bwd_rows<T, K, D, 3, A, LN, EP, 640>
                        : norm_bwd_rows<T, K, D, 4, A, LN, EP, 640>;
    }
  }
  if constexpr (!LN && EP == kEpiNone && D == 1 && K == 4 && Vec<T>::N == 8 && A) {
    if (pl.lacc) {
      if (pl.PF != 1 || pl.W > 16) return hipErrorInvalidValue;
      kern = norm_bwd_rows<T, K, D, 1, A, LN, EP, 1024, false, true>;
    }
  } else {
    if (pl.lacc) return hipErrorInvalidValue;
  }
  // RoPE with several chunks per lane: when a lane's chunks sit at the same
  // offset in their heads, one set of angles per row (the two-chunk kernel
  // spilled with one per chunk)
  if constexpr (EP == kEpiRope && K > 1 && D == 1) {
    if ((64 * pl.W * Vec<T>::N) % ra.head_dim == 0)
      kern = pl.PF == 2 ? norm_bwd_rows<T, K, D, 2, A, LN, EP, 1024, true>
                        : norm_bwd_rows<T, K, D, 1, A, LN, EP, 1024, true>;
  }
  hipLaunchKernelGGL(kern, dim3(pl.P), dim3(64 * pl.W), 0, st, static_cast<const T*>(dy),
                     static_cast<const T*>(x), static_cast<const T*>(w),
                     static_cast<const T*>(beta), mean, rstat, static_cast<T*>(dx), part,
                     part_stride, rows, n, w_add, ra);
  return hipGetLastError();
}

// (K, D) pairs with K * D <= 8: the row batch stays within the register
// budget of a 1024-thread workgroup.
template <typename T, bool A, bool LN, int EP>
hipError_t launch_bwd_a(const BwdPlan& pl, const void* dy, const void* x, const void* w,
                        const void* beta, const float* mean, const float* rstat, void* dx,
                        float* part, int64_t rows, int n, float w_add, const RopeArgs& ra,
                        hipStream_t st) {
  const int key = pl.K * 16 + pl.D;
  switch (key) {
#define NR_CASE(KK, DD)                                                                          \
  case KK * 16 + DD:                                                                             \
    return launch_bwd_kd<T, KK, DD, A, LN, EP>(pl, dy, x, w, beta, mean, rstat, dx, part, rows, n, \
                                               w_add, ra, st);
    NR_CASE(1, 1) NR_CASE(1, 2) NR_CASE(1, 4) NR_CASE(1, 8)
    NR_CASE(2, 1) NR_CASE(2, 2) NR_CASE(2, 4)
    NR_CASE(4, 1) NR_CASE(4, 2)
    NR_CASE(8, 1)
#undef NR_CASE
    default: return hipErrorInvalidValue;
  }
}

template <typename T, bool LN, int EP>
hipError_t launch_bwd_t(const BwdPlan& pl, const void* dy, const void* x, const void* w,
                        const void* beta, const float* mean, const float* rstat, void* dx,
                        float* part, int64_t rows, int n, float w_add, const RopeArgs& ra,
                        hipStream_t st) {
  return pl.aligned ? launch_bwd_a<T, true, LN, EP>(pl, dy, x, w, beta, mean, rstat, dx, part, rows, n, w_add, ra, st)
                    : launch_bwd_a<T, false, LN, EP>(pl, dy, x, w, beta, mean, rstat, dx, part, rows, n, w_add, ra, st);
}


// One translation unit instantiates each (type, operator, epilogue)
// combination, so the build compiles them in parallel.
#define NR_BWD_INSTANTIATE(T, LN, EPI)                                                         \
  template hipError_t launch_bwd_t<T, LN, EPI>(const BwdPlan&, const void*, const void*,       \
                                               const void*, const void*, const float*,          \
                                               const float*, void*, float*, int64_t, int, float, \
                                               const RopeArgs&, hipStream_t);

}  // namespace nr
