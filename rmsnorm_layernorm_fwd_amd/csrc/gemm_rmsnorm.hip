// gemm_rmsnorm.hip -- RMSNorm (or LayerNorm) folded into the following
// linear layer: out = Norm(x) W^T, with the normalised activation never
// written to HBM.
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
// gfx950 mapping, two kernels with v_mfma_f32_32x32x16_bf16:
//  - tile256: a 256 x 256 output tile per 8-wave workgroup (2 waves per
//    SIMD, each wave 128 x 64, 4 x 2 MFMA tiles) when N is a multiple of
//    256.  The row
//    statistics come from a light pass over x (row_inv_rms_kernel) and the
//    norm weight is folded into W beforehand (fold_norm_weight_kernel,
//    w'_k W[n][k] rounded once to bf16, into a caller workspace), so both
//    operands go from HBM straight into LDS with buffer_load ... lds (no
//    VGPR staging, no VALU on the way): two LDS stages of K 64, the next
//    stage's loads in flight while the matrix cores work on the current
//    one, one barrier per stage, placed before the stage's last 8 MFMAs so
//    that they cover the next stage's first operand reads.  LDS rows are
//    128 bytes, 16-byte chunk
//    index XOR-swizzled by the row so the operand reads of 16 consecutive
//    rows hit distinct banks.  r_m scales the accumulators in the epilogue.
//  - tile128: a 128 x 128 tile per 4-wave workgroup for the other N (a
//    multiple of 128); operands staged through VGPRs, W
//    scaled by the norm weight on the way into LDS, the row sums of squares
//    taken from the staged x (no workspace).
// Both number the workgroups so that each of the 8 XCDs (own L2 each) works
// through a contiguous run of tiles, and write the output tile through LDS
// for 16-byte stores.
#include <algorithm>

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
rmsnorm_linear_tile128_kernel(const bf16* __restrict__ x, const bf16* __restrict__ wn,
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

// ---- tile256: folded weight, direct-to-LDS operands ------------------------

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int kBig = 256;                       // output tile edge
constexpr int kBigThreads = 512;                // 8 waves, 2 per SIMD
constexpr int kBigABytes = kBig * BK * 2;       // one operand of one stage (32 KiB)
constexpr int kBigStage = 2 * kBigABytes;       // x and W of one K step (64 KiB)
constexpr int kGroupM = 8;                      // row tiles per group of the tile order

struct BigLoads {
  rsrc_t xr, wr;  // x rows of the tile, W rows of the tile
  int v0, v1;     // per-lane byte offsets (even / odd load instruction)
  int wave;       // wave index, wave-uniform
  int K;
};

// The loads of one K step into stage `dst`: 64 instructions of 1 KiB, 8 per
// wave, 4 of x and 4 of W; instruction j = 4 wave + q % 4 covers rows 8 j ..
// 8 j + 7, lane -> row 8 j + lane / 8, 16-byte chunk lane % 8 of the row's
// LDS slot.  A lane's LDS slot is fixed by the instruction (lane * 16 from
// the wave-uniform base), so the swizzle is applied on the global side: the
// slot holds logical chunk (lane % 8) ^ swz(row), swz(row) = (row & 7) ^
// ((row >> 3) & 1) = (lane / 8) ^ (j & 1).  Rows past M read out of range
// (zero, or stale LDS): they only feed output rows that are never stored.
// The restrict qualifier gives these LDS writes an alias scope of their own,
// so the compiler's wait-count pass does not make the other stage's operand
// reads wait for them.
__device__ __forceinline__ void big_load_stage(lds_char* __restrict__ dst, const BigLoads& c,
                                               int k0) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int j = 4 * c.wave + (q & 3);
    lds_char* d = dst + (q >> 2) * kBigABytes + j * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        (q >> 2) ? c.wr : c.xr, reinterpret_cast<__attribute__((address_space(3))) void*>(d), 16,
        (q & 1) ? c.v1 : c.v0, k0 * 2 + 8 * j * c.K * 2, 0, 0);
  }
}

// The 8 MFMAs of one sub-step of 16 (4 x 2 tiles of 32 x 32), at raised
// wave priority so that the SIMD's other wave fills the gaps rather than
// delaying the matrix work.
__device__ __forceinline__ void big_mfma(const u32x4 (&a)[4], const u32x4 (&b)[2],
                                         f32x16 (&acc)[4][2]) {
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_frag(a[i]), as_frag(b[j]), acc[i][j],
                                                         0, 0, 0);
  __builtin_amdgcn_s_setprio(0);
}

// One K step of 64 on stage `cur` (4 sub-steps of 16), entered right after
// the barrier that completed `cur`.  Each wave owns a 128 x 64 block of the
// output (4 x 2 MFMA tiles).  Order: the next step's loads into `nxt`; the
// operand reads of sub-step 0, covered by the previous step's sub-step 3
// MFMAs (`prev`: operands still in buffer 1); then sub-steps 0..2, each
// with the next one's reads in flight.  The step ends at the barrier, once
// sub-step 3's operands are in registers: its MFMAs open the next step, so
// the matrix cores have work while every wave waits for its first reads of
// the new stage.  The barrier also frees `cur` for the loads issued next.
__device__ __forceinline__ void big_step(const lds_char* __restrict__ cur, lds_char* __restrict__ nxt,
                                         const BigLoads& c, int k_next, bool load, bool prev,
                                         int arow, int brow, const int (&ko)[4],
                                         f32x16 (&acc)[4][2], u32x4 (&af)[2][4],
                                         u32x4 (&bfr)[2][2]) {
  if (load) big_load_stage(nxt, c, k_next);
  __builtin_amdgcn_sched_barrier(0);
  auto read = [&](int ks, int b) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[b][i] = *reinterpret_cast<const lds_u32x4*>(cur + (arow + i * 32) * 128 + ko[ks]);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      bfr[b][j] = *reinterpret_cast<const lds_u32x4*>(cur + kBigABytes + (brow + j * 32) * 128 + ko[ks]);
  };
  read(0, 0);
  if (prev) {
    big_mfma(af[1], bfr[1], acc);
    // scheduling: the 6 operand reads, then the 8 MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  }
#pragma unroll
  for (int ks = 0; ks < 3; ++ks) {
    const int b = ks & 1;
    read(ks + 1, b ^ 1);
    big_mfma(af[b], bfr[b], acc);
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  }
  // this wave's loads into `nxt` have landed, its reads of `cur` are done
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();
}

// LN: the LayerNorm form of the epilogue, out = r_m (acc - mu_m c_n) + d_n
// (mu, c, d as described at launch_layernorm_linear); otherwise
// out = r_m acc.
template <bool LN>
__global__ void __launch_bounds__(kBigThreads)
norm_linear_tile256_kernel(const bf16* __restrict__ x, const bf16* __restrict__ W,
                           bf16* __restrict__ out, const float* __restrict__ rin,
                           const float* __restrict__ mu, const float* __restrict__ cn,
                           const float* __restrict__ dn, int M, int N, int K, int tiles_m,
                           int tiles_n) {
  // two LDS stages as separate arrays: the loads into one and the operand
  // reads of the other are then provably disjoint
  __shared__ __align__(1024) char st0[kBigStage];
  __shared__ __align__(1024) char st1[kBigStage];
  __shared__ float rrow[kBig];
  __shared__ float mrow[LN ? kBig : 1], ccol[LN ? kBig : 1], dcol[LN ? kBig : 1];

  // tile order: XCD (workgroup id mod 8) takes a contiguous run of tile
  // numbers; numbers go through groups of kGroupM row tiles, column-major
  // inside a group, so the tiles running at once share x and W panels in L2
  const int T = gridDim.x;
  int L = blockIdx.x;
  if (T % 8 == 0) L = (L % 8) * (T / 8) + L / 8;
  const int gsize = kGroupM * tiles_n;
  const int grp = L / gsize, rem = L - grp * gsize;
  const int rows_g = min(kGroupM, tiles_m - grp * kGroupM);
  const int mt = grp * kGroupM + rem % rows_g, nt = rem / rows_g;
  const int m0 = mt * kBig, n0 = nt * kBig;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 2, wn_ = wave & 3;  // 2 x 4 waves of 128 x 64 outputs
  const int xrows = min(M - m0, kBig);
  BigLoads c;
  c.xr = make_rsrc(x + static_cast<int64_t>(m0) * K, static_cast<uint32_t>(xrows * K * 2));
  c.wr = make_rsrc(W + static_cast<int64_t>(n0) * K, static_cast<uint32_t>(kBig * K * 2));
  c.wave = __builtin_amdgcn_readfirstlane(wave);
  const int lr = lane >> 3, pc = lane & 7;
  c.v0 = lr * K * 2 + 16 * (pc ^ lr);
  c.v1 = lr * K * 2 + 16 * (pc ^ lr ^ 1);
  c.K = K;
  if (t < kBig) rrow[t] = t < xrows ? rin[m0 + t] : 0.0f;
  if constexpr (LN) {
    if (t < kBig) {
      mrow[t] = t < xrows ? mu[m0 + t] : 0.0f;
      ccol[t] = cn[n0 + t];
      dcol[t] = dn != nullptr ? dn[n0 + t] : 0.0f;
    }
  }

  // operand reads: lane l takes A row (and B column) l % 32 of each 32-tile,
  // k chunk 2 ks + l / 32 of the step, at physical chunk ^ swz(row)
  const int fr = lane & 31, h = lane >> 5;
  const int sw = (fr & 7) ^ ((fr >> 3) & 1);
  int ko[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) ko[ks] = ((2 * ks + h) ^ sw) * 16;
  const int arow = wm * 128 + fr, brow = wn_ * 64 + fr;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  lds_char* const l0 = (lds_char*)st0;  // generic -> LDS address space
  lds_char* const l1 = (lds_char*)st1;
  const int nk = K / BK;
  big_load_stage(l0, c, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // two steps per trip so that each stage is a fixed array
  u32x4 af[2][4], bfr[2][2];
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {
    big_step(l0, l1, c, (kt + 1) * BK, true, kt > 0, arow, brow, ko, acc, af, bfr);
    big_step(l1, l0, c, (kt + 2) * BK, kt + 2 < nk, true, arow, brow, ko, acc, af, bfr);
  }
  if (kt < nk) big_step(l0, l1, c, 0, false, kt > 0, arow, brow, ko, acc, af, bfr);
  big_mfma(af[1], bfr[1], acc);  // the last step's sub-step 3
  __syncthreads();  // the stages take the output tile

  // scaled accumulators -> bf16 output tile: rows of row half wm in stage
  // array wm (128 rows x 32 chunks of 16 bytes), chunk index XOR 4 (bit 2 of
  // the row) so the two rows of one 2-byte write use different banks.
  // Accumulator e of MFMA tile (i, j): row 8 (e / 4) + 4 (l / 32) + e % 4,
  // column l % 32.
  {
    uint16_t* Cs = reinterpret_cast<uint16_t*>(wm == 0 ? st0 : st1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const int rl = i * 32 + 8 * (e / 4) + 4 * h + (e % 4);
          const int cc = wn_ * 64 + j * 32 + fr;
          const int r0 = wm * 128 + rl;
          float v0, v1;
          if constexpr (LN) {
            v0 = fmaf(acc[i][j][e] - mrow[r0] * ccol[cc], rrow[r0], dcol[cc]);
            v1 = fmaf(acc[i][j][e + 1] - mrow[r0 + 1] * ccol[cc], rrow[r0 + 1], dcol[cc]);
          } else {
            v0 = acc[i][j][e] * rrow[r0];
            v1 = acc[i][j][e + 1] * rrow[r0 + 1];
          }
          const uint32_t p = pack_bf16x2(v0, v1);
          const int s0 = ((rl >> 2) & 1) << 2, s1 = (((rl + 1) >> 2) & 1) << 2;
          Cs[rl * kBig + (((cc >> 3) ^ s0) << 3) + (cc & 7)] = static_cast<uint16_t>(p & 0xffffu);
          Cs[(rl + 1) * kBig + (((cc >> 3) ^ s1) << 3) + (cc & 7)] = static_cast<uint16_t>(p >> 16);
        }
  }
  __syncthreads();
  // 16-byte stores; rows past M dropped by the buffer range
  const rsrc_t orr = make_rsrc(out + static_cast<int64_t>(m0) * N,
                               static_cast<uint32_t>(xrows * N * 2));
#pragma unroll 4
  for (int q = t; q < kBig * 32; q += kBigThreads) {
    const int row = q >> 5, ch = q & 31, rl = row & 127;
    const uint16_t* Cs = reinterpret_cast<const uint16_t*>(row < 128 ? st0 : st1);
    const u32x4 v = *reinterpret_cast<const u32x4*>(Cs + rl * kBig + ((ch ^ (((rl >> 2) & 1) << 2)) << 3));
    __builtin_amdgcn_raw_buffer_store_b128(v, orr, (row * N + n0 + 8 * ch) * 2, 0, kStream);
  }
}

// Row statistics of the tile256 path: r_m = 1/sqrt(mean_k x[m][k]^2 + eps),
// one wave per row, fp32 sums of 16-byte chunks.
__global__ void __launch_bounds__(256)
row_inv_rms_kernel(const bf16* __restrict__ x, float* __restrict__ r, int M, int K, float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= M) return;
  const rsrc_t xr = make_rsrc(x + static_cast<int64_t>(row) * K, static_cast<uint32_t>(K) * 2u);
  float s = 0.0f;
  for (int c = lane; c < K / 8; c += 64) {
    float f[8];
    unpack<bf16>(__builtin_amdgcn_raw_buffer_load_b128(xr, c * 16, 0, kStream), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(f[e], f[e], s);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) r[row] = rsqrtf(s / static_cast<float>(K) + eps);
}

// Row statistics of the LayerNorm form: mean_m and rstd_m = 1/sqrt(var_m +
// eps) with the biased variance, one wave per row, fp32.  The variance is
// the mean of the centred squares, a second pass over the row: with
// CPL > 0 over the row kept in registers (CPL 16-byte chunks per lane, rows
// of up to 512 CPL elements: one read of x from HBM), with CPL == 0 over
// the row read again (longer rows; the second read mostly misses the cache).
template <int CPL>
__global__ void __launch_bounds__(256)
row_mean_rstd_kernel(const bf16* __restrict__ x, float* __restrict__ mean,
                     float* __restrict__ rstd, int M, int K, float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= M) return;
  const int chunks = K / 8;
  const rsrc_t xr = make_rsrc(x + static_cast<int64_t>(row) * K, static_cast<uint32_t>(K) * 2u);
  float s = 0.0f, q = 0.0f, mu;
  if constexpr (CPL > 0) {
    // chunks past the row read as 0 (buffer range) and are left out of the
    // centred squares
    u32x4 v[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, (lane + 64 * i) * 16, 0, kStream);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      float f[8];
      unpack<bf16>(v[i], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += f[e];
    }
    mu = wave_sum(s) / static_cast<float>(K);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      if (lane + 64 * i >= chunks) break;
      float f[8];
      unpack<bf16>(v[i], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = f[e] - mu;
        q = fmaf(d, d, q);
      }
    }
  } else {
    for (int c = lane; c < chunks; c += 64) {
      float f[8];
      unpack<bf16>(__builtin_amdgcn_raw_buffer_load_b128(xr, c * 16, 0, 0), f);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += f[e];
    }
    mu = wave_sum(s) / static_cast<float>(K);
    for (int c = lane; c < chunks; c += 64) {
      float f[8];
      unpack<bf16>(__builtin_amdgcn_raw_buffer_load_b128(xr, c * 16, 0, kStream), f);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = f[e] - mu;
        q = fmaf(d, d, q);
      }
    }
  }
  const float r = rsqrtf(wave_sum(q) / static_cast<float>(K) + eps);
  if (lane == 0) {
    mean[row] = mu;
    rstd[row] = r;
  }
}

// Per output column n of the LayerNorm form, one wave per row of W:
//   Wf[n][k] = bf16(gamma_k W[n][k])     (written when gamma is given)
//   c_n = sum_k Wf[n][k]                 (the weight the matrix cores use)
//   d_n = sum_k beta_k W[n][k]           (0 without beta)
// fp32 sums, each lane over its chunks in order, then the wave sum.
__global__ void __launch_bounds__(256)
fold_ln_weight_kernel(const bf16* __restrict__ gamma, const bf16* __restrict__ beta,
                      const bf16* __restrict__ W, bf16* __restrict__ Wf, float* __restrict__ cn,
                      float* __restrict__ dn, int N, int K) {
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (n >= N) return;
  const int64_t row = static_cast<int64_t>(n) * K;
  float c = 0.0f, d = 0.0f;
  for (int k8 = lane; k8 < K / 8; k8 += 64) {
    float w[8], g[8], b[8];
    unpack<bf16>(*reinterpret_cast<const u32x4*>(W + row + 8 * k8), w);
    if (gamma != nullptr) {
      unpack<bf16>(*reinterpret_cast<const u32x4*>(gamma + 8 * k8), g);
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = w[e] * g[e];
      const u32x4 packed = pack<bf16>(f);
      *reinterpret_cast<u32x4*>(Wf + row + 8 * k8) = packed;
      unpack<bf16>(packed, f);  // the rounded weight, as the matrix cores see it
#pragma unroll
      for (int e = 0; e < 8; ++e) c += f[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) c += w[e];
    }
    if (beta != nullptr) {
      unpack<bf16>(*reinterpret_cast<const u32x4*>(beta + 8 * k8), b);
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(b[e], w[e], d);
    }
  }
  c = wave_sum(c);
  d = wave_sum(d);
  if (lane == 0) {
    cn[n] = c;
    dn[n] = d;
  }
}

// W_folded[n][k] = bf16(W[n][k] (w_k + w_add)), 8 elements per lane.
__global__ void __launch_bounds__(256)
fold_norm_weight_kernel(const bf16* __restrict__ wn, const bf16* __restrict__ W,
                        bf16* __restrict__ Wf, int64_t chunks, int kchunks, float w_add) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t c = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; c < chunks;
       c += stride) {
    const int kc = static_cast<int>(c % kchunks);
    float a[8], b[8];
    unpack<bf16>(*reinterpret_cast<const u32x4*>(W + 8 * c), a);
    unpack<bf16>(*reinterpret_cast<const u32x4*>(wn + 8 * kc), b);
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] *= b[e] + w_add;
    *reinterpret_cast<u32x4*>(Wf + 8 * c) = pack<bf16>(a);
  }
}

template <int TM, int TN>
hipError_t launch_tile(const void* x, const void* wn, const void* W, void* out, float* inv_rms,
                       int M, int N, int K, float eps, float w_add, hipStream_t st) {
  constexpr int BM = 64 * TM, BN = 64 * TN;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = N / BN;
  const int64_t tiles = static_cast<int64_t>(tiles_m) * tiles_n;
  hipLaunchKernelGGL((rmsnorm_linear_tile128_kernel<TM, TN>), dim3(static_cast<unsigned>(tiles)),
                     dim3(kThreads), 0, st, static_cast<const bf16*>(x),
                     static_cast<const bf16*>(wn), static_cast<const bf16*>(W),
                     static_cast<bf16*>(out), inv_rms, M, N, K, eps, w_add, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fold_norm_weight(const void* wn, const void* W, void* Wf, int64_t N, int K,
                                   float w_add, hipStream_t st) {
  const int64_t chunks = N * K / 8;
  const int64_t blocks = std::min<int64_t>((chunks + 255) / 256, 4096);
  hipLaunchKernelGGL(fold_norm_weight_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                     static_cast<const bf16*>(wn), static_cast<const bf16*>(W),
                     static_cast<bf16*>(Wf), chunks, K / 8, w_add);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_linear(const void* x, const void* wn, const void* W, void* out,
                                 float* inv_rms, void* ws, int M, int N, int K, float eps,
                                 float w_add, int tile, hipStream_t st) {
  if (tile != 2) return launch_tile<2, 2>(x, wn, W, out, inv_rms, M, N, K, eps, w_add, st);
  // workspace: r (M fp32, when inv_rms is NULL), then the folded weight
  float* r = inv_rms != nullptr ? inv_rms : static_cast<float*>(ws);
  void* wfold = static_cast<char*>(ws) + linear_rows_bytes(M);
  hipLaunchKernelGGL(row_inv_rms_kernel, dim3(static_cast<unsigned>((M + 3) / 4)), dim3(256), 0, st,
                     static_cast<const bf16*>(x), r, M, K, eps);
  const void* Wop = W;
  if (wn != nullptr) {
    const hipError_t e = launch_fold_norm_weight(wn, W, wfold, N, K, w_add, st);
    if (e != hipSuccess) return e;
    Wop = wfold;
  }
  const int tiles_m = (M + kBig - 1) / kBig, tiles_n = N / kBig;
  hipLaunchKernelGGL(norm_linear_tile256_kernel<false>,
                     dim3(static_cast<unsigned>(static_cast<int64_t>(tiles_m) * tiles_n)),
                     dim3(kBigThreads), 0, st, static_cast<const bf16*>(x),
                     static_cast<const bf16*>(Wop), static_cast<bf16*>(out), r, nullptr, nullptr,
                     nullptr, M, N, K, tiles_m, tiles_n);
  return hipGetLastError();
}

// LayerNorm folded into the linear layer:
//   out[m][n] = sum_k ((x[m][k] - mu_m) r_m gamma_k + beta_k) W[n][k]
//             = r_m (sum_k x[m][k] Wf[n][k] - mu_m c_n) + d_n
// with Wf = bf16(gamma W), c_n = sum_k Wf[n][k] (so that the centring is
// exact relative to the weight the matrix cores use) and d_n = sum_k beta_k
// W[n][k].  The row statistics go to mean / rstd (or the workspace), the
// column terms and the folded weight to the workspace; then the same
// 256 x 256 matrix-core kernel with the LayerNorm epilogue.
hipError_t launch_layernorm_linear(const void* x, const void* gamma, const void* beta,
                                   const void* W, void* out, float* mean, float* rstd, void* ws,
                                   int M, int N, int K, float eps, hipStream_t st) {
  char* p = static_cast<char*>(ws);
  float* mu = mean != nullptr ? mean : reinterpret_cast<float*>(p);
  p += linear_rows_bytes(M);
  float* rs = rstd != nullptr ? rstd : reinterpret_cast<float*>(p);
  p += linear_rows_bytes(M);
  float* cn = reinterpret_cast<float*>(p);
  p += linear_rows_bytes(N);
  float* dn = reinterpret_cast<float*>(p);
  p += linear_rows_bytes(N);
  bf16* wf = reinterpret_cast<bf16*>(p);
  // the row in registers when it fits 4, 10 or 16 chunks per lane (the
  // fewest that cover it), else read twice
  const int cpl = (K / 8 + 63) / 64;
  auto stats = cpl <= 4    ? row_mean_rstd_kernel<4>
               : cpl <= 10 ? row_mean_rstd_kernel<10>
               : cpl <= 16 ? row_mean_rstd_kernel<16>
                           : row_mean_rstd_kernel<0>;
  hipLaunchKernelGGL(stats, dim3(static_cast<unsigned>((M + 3) / 4)), dim3(256), 0, st,
                     static_cast<const bf16*>(x), mu, rs, M, K, eps);
  hipLaunchKernelGGL(fold_ln_weight_kernel, dim3(static_cast<unsigned>((N + 3) / 4)), dim3(256), 0,
                     st, static_cast<const bf16*>(gamma), static_cast<const bf16*>(beta),
                     static_cast<const bf16*>(W), wf, cn, dn, N, K);
  const bf16* Wop = gamma != nullptr ? wf : static_cast<const bf16*>(W);
  const int tiles_m = (M + kBig - 1) / kBig, tiles_n = N / kBig;
  hipLaunchKernelGGL(norm_linear_tile256_kernel<true>,
                     dim3(static_cast<unsigned>(static_cast<int64_t>(tiles_m) * tiles_n)),
                     dim3(kBigThreads), 0, st, static_cast<const bf16*>(x), Wop,
                     static_cast<bf16*>(out), rs, mu, cn, dn, M, N, K, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace nr
