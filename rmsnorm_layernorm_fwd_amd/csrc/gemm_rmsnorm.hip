// gemm_rmsnorm.hip -- RMSNorm folded into the following linear layer:
// out = RMSNorm(x) W^T, with the normalised activation never written to HBM.
//
// The pages fuse element-wise work into its neighbours to save memory round
// trips (Helios 性能优化全解析, 内核一 FlashNorm and the closing advice to
// optimise memory rather than arithmetic); folding the norm into the GEMM
// that consumes it removes the activation's write and re-read.  Since
//   out[m][n] = r_m sum_k x[m][k] w'_k W[n][k],   r_m = 1/sqrt(mean_k x[m][k]^2 + eps),
// the kernel multiplies the raw x (exact in bf16) by W scaled with the norm
// weight (w'_k W[n][k], rounded once to bf16 as it is staged), accumulates
// each row's sum of squares from the same x tiles it feeds to the matrix
// cores, and applies r_m to the fp32 accumulators in the epilogue.
//
// gfx950 mapping: a 256-lane workgroup computes a 128 x 128 or 256 x 256
// output tile with v_mfma_f32_32x32x16_bf16, each wave a quarter of it
// (2 x 2 or 4 x 4 MFMA tiles; the large tile halves the LDS operand reads
// per MFMA and keeps its accumulators in the AGPRs).  K advances 64 at a
// time: the next step's x and W chunks are loaded into registers while the
// matrix cores work on the current step from LDS.  LDS rows are padded to 72
// elements so that the 16-byte operand reads of 16 consecutive rows land on
// distinct banks.  Workgroups are numbered so that
// each of the 8 XCDs (own L2 each) works through a contiguous run of tiles
// that share x rows.  The output tile goes through LDS for 16-byte stores.
#include "nr_device.hpp"
#include "nr_internal.hpp"

namespace nr {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row (elements)
constexpr int kThreads = 256;

__device__ __forceinline__ bf16x8_t as_frag(const u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// TM x TN MFMA tiles of 32 x 32 per wave; the 4 waves tile the workgroup's
// (64 TM) x (64 TN) output 2 x 2.
template <int TM, int TN>
__global__ void __launch_bounds__(kThreads)
rmsnorm_linear_kernel(const bf16* __restrict__ x, const bf16* __restrict__ wn,
                      const bf16* __restrict__ W, bf16* __restrict__ out, float* inv_rms, int M,
                      int N, int K, float eps, float w_add, int tiles_n) {
  constexpr int BM = 64 * TM, BN = 64 * TN;
  constexpr int CA = BM / 32, CB = BN / 32;  // 16-byte chunks per thread per step (A, B)
  constexpr int LDC = BN + 8;                // padded output-tile row (elements)
  constexpr int LDS_AB = (BM + BN) * LDK, LDS_C = BM * LDC;
  // A (x) and B (scaled W) tiles of one K step; reused for the output tile
  __shared__ __align__(16) uint16_t lds[LDS_AB > LDS_C ? LDS_AB : LDS_C];
  __shared__ float rrow[BM];
  uint16_t* As = lds;
  uint16_t* Bs = lds + BM * LDK;

  // tile numbering: XCD xcd (= workgroup id mod 8) takes a contiguous run
  const int T = gridDim.x;
  int b = blockIdx.x;
  if (T % 8 == 0) b = (b % 8) * (T / 8) + b / 8;
  const int mt = b / tiles_n, nt = b - (b / tiles_n) * tiles_n;
  const int m0 = mt * BM, n0 = nt * BN;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn_ = wave & 1;

  // staging: thread t moves chunks t + 256 i of each tile: row (t >> 3) +
  // 32 i, 16-byte chunk t & 7 of the row's 64 elements
  const int srow = t >> 3, skc = t & 7;
  const uint32_t xbytes_row = static_cast<uint32_t>(K) * 2u;
  // x rows past M read as 0 (buffer range), W has whole tiles
  const int64_t xrows = static_cast<int64_t>(M - m0 < BM ? M - m0 : BM);
  const rsrc_t xr = make_rsrc(x + static_cast<int64_t>(m0) * K,
                              static_cast<uint32_t>(xrows * K * 2));
  const rsrc_t wr = make_rsrc(W + static_cast<int64_t>(n0) * K, static_cast<uint32_t>(BN) * xbytes_row);
  const rsrc_t nr_ = make_rsrc(wn, wn != nullptr ? xbytes_row : 0u);

  u32x4 xa[CA], wb[CB], wnc;
  float ss[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) ss[i] = 0.0f;
  auto load_step = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CA; ++i)
      xa[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, ((srow + 32 * i) * K + k0 + 8 * skc) * 2, 0,
                                                    kStream);
#pragma unroll
    for (int i = 0; i < CB; ++i)
      wb[i] = __builtin_amdgcn_raw_buffer_load_b128(wr, ((srow + 32 * i) * K + k0 + 8 * skc) * 2, 0,
                                                    0);
    wnc = __builtin_amdgcn_raw_buffer_load_b128(nr_, (k0 + 8 * skc) * 2, 0, 0);
  };
  auto stage = [&]() {
    float wv[8];
    unpack<bf16>(wnc, wv);
#pragma unroll
    for (int e = 0; e < 8; ++e) wv[e] = (wn != nullptr) ? wv[e] + w_add : 1.0f;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      float xv[8];
      unpack<bf16>(xa[i], xv);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss[i] = fmaf(xv[e], xv[e], ss[i]);
      *reinterpret_cast<u32x4*>(As + (srow + 32 * i) * LDK + 8 * skc) = xa[i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      float bv[8];
      unpack<bf16>(wb[i], bv);
#pragma unroll
      for (int e = 0; e < 8; ++e) bv[e] *= wv[e];
      *reinterpret_cast<u32x4*>(Bs + (srow + 32 * i) * LDK + 8 * skc) = pack<bf16>(bv);
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // operand rows of this lane: A row (and B column) l % 32 of each 32-tile,
  // k offset 8 (l / 32) within each 16-wide k step
  const int fr = lane & 31, fk = 8 * (lane >> 5);

  load_step(0);
  for (int k0 = 0; k0 < K; k0 += BK) {
    stage();
    __syncthreads();
    if (k0 + BK < K) load_step(k0 + BK);  // in flight during the MFMAs
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = as_frag(*reinterpret_cast<const u32x4*>(As + (wm * 32 * TM + i * 32 + fr) * LDK + ks + fk));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = as_frag(*reinterpret_cast<const u32x4*>(Bs + (wn_ * 32 * TN + j * 32 + fr) * LDK + ks + fk));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();  // the tiles are restaged next step
  }

  // each row's sum of squares: the 8 lanes of a row group (t & 7) add up
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    float v = ss[i];
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    if (skc == 0) {
      const float r = rsqrtf(v / static_cast<float>(K) + eps);
      rrow[srow + 32 * i] = r;
      const int m = m0 + srow + 32 * i;
      if (nt == 0 && inv_rms != nullptr && m < M) inv_rms[m] = r;
    }
  }
  __syncthreads();

  // scaled accumulators -> bf16 output tile in LDS.  Accumulator e of MFMA
  // tile (i, j) is row 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32.
  uint16_t* Cs = lds;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const int r0 = wm * 32 * TM + i * 32 + 8 * (e / 4) + 4 * (lane >> 5) + (e % 4);
        const int c = wn_ * 32 * TN + j * 32 + fr;
        const uint32_t p =
            pack_bf16x2(acc[i][j][e] * rrow[r0], acc[i][j][e + 1] * rrow[r0 + 1]);
        Cs[r0 * LDC + c] = static_cast<uint16_t>(p & 0xffffu);
        Cs[(r0 + 1) * LDC + c] = static_cast<uint16_t>(p >> 16);
      }
  __syncthreads();

  // 16-byte stores: BM rows x BN / 8 chunks; rows past M dropped
  const rsrc_t orr = make_rsrc(out + static_cast<int64_t>(m0) * N,
                               static_cast<uint32_t>(xrows * N * 2));
  constexpr int CPR = BN / 8;  // chunks per output row
#pragma unroll 4
  for (int c = t; c < BM * CPR; c += kThreads) {
    const int row = c / CPR, ch = c % CPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(Cs + row * LDC + 8 * ch);
    __builtin_amdgcn_raw_buffer_store_b128(v, orr, (row * N + n0 + 8 * ch) * 2, 0, kStream);
  }
}

template <int TM, int TN>
hipError_t launch_tile(const void* x, const void* wn, const void* W, void* out, float* inv_rms,
                       int M, int N, int K, float eps, float w_add, hipStream_t st) {
  constexpr int BM = 64 * TM, BN = 64 * TN;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = N / BN;
  const int64_t tiles = static_cast<int64_t>(tiles_m) * tiles_n;
  hipLaunchKernelGGL((rmsnorm_linear_kernel<TM, TN>), dim3(static_cast<unsigned>(tiles)),
                     dim3(kThreads), 0, st, static_cast<const bf16*>(x),
                     static_cast<const bf16*>(wn), static_cast<const bf16*>(W),
                     static_cast<bf16*>(out), inv_rms, M, N, K, eps, w_add, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm_linear(const void* x, const void* wn, const void* W, void* out,
                                 float* inv_rms, int M, int N, int K, float eps, float w_add,
                                 int tile, hipStream_t st) {
  switch (tile) {
    case 2: return launch_tile<2, 4>(x, wn, W, out, inv_rms, M, N, K, eps, w_add, st);
    case 3: return launch_tile<4, 2>(x, wn, W, out, inv_rms, M, N, K, eps, w_add, st);
    case 4: return launch_tile<4, 4>(x, wn, W, out, inv_rms, M, N, K, eps, w_add, st);
    default: return launch_tile<2, 2>(x, wn, W, out, inv_rms, M, N, K, eps, w_add, st);
  }
}

}  // namespace nr
