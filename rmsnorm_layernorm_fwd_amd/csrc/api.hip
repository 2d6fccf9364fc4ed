// api.hip -- the C ABI of libnormrope.so (declared in include/normrope.h):
// host-side argument checks, launch-shape selection and kernel dispatch.
//
// Launch-shape selection plays the part of the pages' block-size heuristic
// (Helios 性能优化全解析, 内核一 FlashNorm: the row length is rounded up and
// the thread count grows with it, few threads for short rows, a full block
// for long ones), re-derived for 64-wide wavefronts: a row that fits in one
// wave's registers (up to 640 16-byte chunks, i.e. 5120 bf16) gets one
// wavefront and no barrier; longer rows get W waves.  Every check runs before
// any HIP call, so a rejected call touches neither the device nor the stream.
#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>

#include "../../include/normrope.h"
#include "nr_internal.hpp"

namespace {

using nr::BwdPlan;
using nr::FwdPlan;
using nr::RopePlan;

// ---- tuning overrides ---------------------------------------------------

enum TuneKey { FWD_W, FWD_K, FWD_R, FWD_J, BWD_W, BWD_K, BWD_D, BWD_P, BWD_ROWS_MIN, BWD_PF,
               ROPE_K, ROPE_WPB, ROPE_GROUPS, GEMM_TILE, FWD_PACK, BWD_PACK, NKEYS };
const char* const kTuneNames[NKEYS] = {"fwd_w", "fwd_k", "fwd_r", "fwd_j", "bwd_w", "bwd_k",
                                       "bwd_d", "bwd_p", "bwd_rows_min", "bwd_pf", "rope_k",
                                       "rope_wpb", "rope_groups", "gemm_tile", "fwd_pack",
                                       "bwd_pack"};
std::atomic<int> g_tune[NKEYS];

int tune(TuneKey k) { return g_tune[k].load(std::memory_order_relaxed); }

thread_local int t_last_hip = 0;

nr_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return NR_OK;
  t_last_hip = static_cast<int>(e);
  return NR_ERR_HIP;
}

constexpr int64_t kMaxChunksPerRow = 16 * 64 * 8;  // 16 waves x 64 lanes x 8 chunks

int elem_bytes(nr_dtype_t dt) { return dt == NR_F32 ? 4 : 2; }
int vec_elems(nr_dtype_t dt) { return dt == NR_F32 ? 4 : 8; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool in_set(int v, const int* set, int n) {
  for (int i = 0; i < n; ++i)
    if (set[i] == v) return true;
  return false;
}

// smallest member of the (ascending) set that is >= need, or 0
int pick_at_least(int64_t need, const int* set, int n) {
  for (int i = 0; i < n; ++i)
    if (set[i] >= need) return set[i];
  return 0;
}

const int kFwdK[] = {1, 2, 4, 5, 6, 8, 10};
const int kBwdK[] = {1, 2, 4, 8};
const int kBwdD[] = {1, 2, 4, 8};
const int kRopeK[] = {1, 2, 4, 5, 6, 8, 10};

// Two byte ranges either coincide exactly or are disjoint.
bool bad_overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  if (a0 == b0 && na == nb) return false;
  return a0 < b0 + nb && b0 < a0 + na;
}

// Two byte ranges share at least one byte (ranges that coincide included).
// Range ends saturate, so a size past the address space cannot wrap.
bool any_overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  const uintptr_t a1 = na > UINTPTR_MAX - a0 ? UINTPTR_MAX : a0 + na;
  const uintptr_t b1 = nb > UINTPTR_MAX - b0 ? UINTPTR_MAX : b0 + nb;
  return a0 < b1 && b0 < a1;
}

// The forward's outputs against its inputs, x against y excepted (in place
// is the caller's choice, checked by the caller): y and the row statistics
// are written while x, the weights and the tables are read.
bool fwd_buffers_disjoint(nr_dtype_t dt, int64_t rows, int64_t n, const void* x, const void* w,
                          const void* beta, const void* y, const float* s0, const float* s1,
                          const float* cos_tab = nullptr, const float* sin_tab = nullptr,
                          size_t tab_bytes = 0) {
  const size_t bytes = static_cast<size_t>(rows * n) * elem_bytes(dt);
  const size_t wb = static_cast<size_t>(n) * elem_bytes(dt);
  const size_t sb = static_cast<size_t>(rows) * sizeof(float);
  struct Range { const void* p; size_t n; };
  const Range read[] = {{x, bytes}, {w, wb}, {beta, wb}, {cos_tab, tab_bytes}, {sin_tab, tab_bytes}};
  const Range written[] = {{y, bytes}, {s0, sb}, {s1, sb}};
  for (int i = 0; i < 3; ++i) {
    for (int j = (i == 0 ? 1 : 0); j < 5; ++j)
      if (any_overlap(written[i].p, written[i].n, read[j].p, read[j].n)) return false;
    for (int j = i + 1; j < 3; ++j)
      if (any_overlap(written[i].p, written[i].n, written[j].p, written[j].n)) return false;
  }
  return true;
}

// The backward's buffers beyond dx against dy and x (checked by the caller):
// dx, the column gradients and the workspace are written while every other
// operand is read, so none of them may share a byte with another operand.
// (The row statistics are read through the scalar cache, which the writes to
// dx would not update.)
bool bwd_buffers_disjoint(nr_dtype_t dt, int64_t rows, int64_t n, const void* dy, const void* x,
                          const void* w, const void* beta, const float* mean, const float* rstat,
                          const void* dx, const float* o0, const float* o1, const void* workspace,
                          size_t workspace_bytes, const float* cos_tab = nullptr,
                          const float* sin_tab = nullptr, size_t tab_bytes = 0) {
  const size_t bytes = static_cast<size_t>(rows * n) * elem_bytes(dt);
  const size_t wb = static_cast<size_t>(n) * elem_bytes(dt);
  const size_t sb = static_cast<size_t>(rows) * sizeof(float);
  const size_t cb = static_cast<size_t>(n) * sizeof(float);
  struct Range { const void* p; size_t n; };
  const Range read[] = {{dy, bytes}, {x, bytes}, {w, wb}, {beta, wb}, {mean, sb}, {rstat, sb},
                        {cos_tab, tab_bytes}, {sin_tab, tab_bytes}};
  const Range written[] = {{dx, bytes}, {o0, cb}, {o1, cb}, {workspace, workspace_bytes}};
  for (int i = 0; i < 4; ++i) {
    // dx may coincide with dy or x (in place): those pairs are the caller's
    for (int j = (i == 0 ? 2 : 0); j < 8; ++j)
      if (any_overlap(written[i].p, written[i].n, read[j].p, read[j].n)) return false;
    for (int j = i + 1; j < 4; ++j)
      if (any_overlap(written[i].p, written[i].n, written[j].p, written[j].n)) return false;
  }
  return true;
}

nr_status_t check_dtype(nr_dtype_t dt) {
  return (dt == NR_F32 || dt == NR_BF16 || dt == NR_F16) ? NR_OK : NR_ERR_DTYPE;
}

nr_status_t check_norm_shape(nr_dtype_t dt, int64_t rows, int64_t n) {
  if (rows < 0 || n < 1) return NR_ERR_SHAPE;
  if (n > nr_norm_n_max(dt)) return NR_ERR_UNSUPPORTED_N;
  if (rows > INT64_MAX / 8 / n) return NR_ERR_SHAPE;
  return NR_OK;
}

enum FwdOp { kFwdRms, kFwdLn, kFwdRmsRope };

nr_status_t plan_fwd(nr_dtype_t dt, int64_t rows, int64_t n, bool aligned, FwdPlan* pl,
                     FwdOp op) {
  const int64_t nchunk = (n + vec_elems(dt) - 1) / vec_elems(dt);
  const int64_t need = (nchunk + 63) / 64;
  // Short rows: a wavefront per row, no barrier.  Rows of 5..16 chunk slots
  // (up to 8192 bf16 / 4096 fp32), two rows per row group so that each
  // weight chunk loaded serves both:
  //   LayerNorm: two waves per row and about 5 chunks per lane, which keeps
  //     the row resident in fewer VGPRs (it holds x, gamma and beta);
  //   RMSNorm (plain or with the RoPE epilogue) on batches of 16384 rows or
  //     more: 2 chunks per lane and as many waves as that needs, i.e. more
  //     waves with fewer loads each; plain RMSNorm also puts two row groups
  //     in a workgroup.  Smaller batches take the LayerNorm shape, whose
  //     fewer, fuller workgroups leave less of a partial last round.
  // Each measured fastest at 5120 bf16 on MI355X (LayerNorm 5.9 TB/s;
  // 65536 rows: RMSNorm 6.05 -> 6.19, RMSNorm + RoPE 5.85 -> 6.1-6.2 TB/s
  // against the two-wave shape; 3840 rows: RMSNorm 15.5 -> 14.8 us the other
  // way round).  Longer rows: up to 8 chunks per lane and as many waves as
  // needed.
  // Aligned rows of at most 32 chunks (256 16-bit or 128 fp32 elements, e.g.
  // a per-head q/k norm): 64 / S rows side by side in a wave, S lanes each,
  // so no lane idles (norm_fwd_packed).  fwd_pack = 1 keeps the wave-per-row
  // kernels; 4..32 forces S.
  if (aligned && nchunk <= 32 && tune(FWD_PACK) != 1) {
    int S = 4;
    while (S < nchunk) S *= 2;
    if (tune(FWD_PACK) > 1) S = tune(FWD_PACK);
    if ((S != 4 && S != 8 && S != 16 && S != 32) || S < nchunk) return NR_ERR_SHAPE;
    *pl = FwdPlan{1, 1, 1, 1, aligned, S};
    return NR_OK;
  }
  int W, K, J = 1, R;
  if (need <= 4) {
    W = 1;
    K = pick_at_least(need, kFwdK, 7);
    R = 4;
    // rows of up to two chunks a lane: two rows a wave (65536 x 256 bf16
    // RMSNorm 18.0 -> 14.9 us, 2621440 x 128 539 -> 403 us; level at 512)
    if (K <= 2) J = 2;
  } else if (need <= 16 && !aligned) {
    // misaligned rows (element-wise loads): one chunk per lane, two rows per
    // row group; the fuller shapes below spilled there (LayerNorm 15360 x
    // 5118 bf16: 219 against 265 us)
    W = static_cast<int>(need);
    K = 1;
    J = 2;
    R = 1;
  } else if (need <= 16 && op != kFwdLn && rows >= 16384) {
    W = static_cast<int>((need + 1) / 2);
    K = 2;
    J = 2;
    R = (op == kFwdRms && W <= 8) ? 2 : 1;
  } else if (need <= 16) {
    W = 2;
    K = pick_at_least((need + 1) / 2, kFwdK, 6);
    if (K <= 5) J = 2;  // one weight load serves two rows
    R = J == 1 ? 2 : 1;
    // Plain RMSNorm on a batch that sixteen-row workgroups cover in one round
    // of about one workgroup per CU (3584..4096 rows on 256 CUs): eight row
    // groups per workgroup, so the whole batch is dispatched as ~240
    // workgroups instead of ~1900 (3840 x 5120 bf16: 14.1-14.3 -> 13.1-13.4 us
    // on two MI355X boxes; LayerNorm and LayerNorm + GeLU measured level or
    // slower with it, and larger batches slower).
    if (op == kFwdRms && J == 2 && rows >= 3584 && rows <= 4096) R = 8;
  } else {
    W = static_cast<int>((need + 7) / 8);
    K = pick_at_least((need + W - 1) / W, kFwdK, 6);  // K <= 8 when W > 1
    R = 1;
  }
  if (tune(FWD_W) > 0) W = tune(FWD_W);
  if (tune(FWD_K) > 0) K = tune(FWD_K);
  if (tune(FWD_R) > 0) R = tune(FWD_R);
  if (tune(FWD_J) > 0) J = tune(FWD_J);
  if (W < 1 || W > 16 || !in_set(K, kFwdK, 7) || (W > 1 && K > 8)) return NR_ERR_SHAPE;
  if (J < 1 || J > 2 || (J == 2 && K > 5)) return NR_ERR_SHAPE;
  if (static_cast<int64_t>(64) * W * K < nchunk) return NR_ERR_SHAPE;
  if (R < 1 || (W == 1 && R > 4) || 64 * W * R > 1024) return NR_ERR_SHAPE;
  *pl = FwdPlan{W, K, R, J, aligned};
  return NR_OK;
}

// The forward launches one workgroup per J*R rows: the grid must fit the
// hardware's 2^31 - 1 workgroups.
bool fwd_grid_ok(int64_t rows, const FwdPlan& pl) {
  const int64_t per = pl.S > 0 ? nr::fwd_packed_rows_per_block(pl.S) : static_cast<int64_t>(pl.J) * pl.R;
  return (rows + per - 1) / per <= INT32_MAX;
}

// Backward of aligned rows of at most 32 chunks (every operator): the lanes
// per row S of the packed kernel (0: the row kernels), and its workgroup count, at least one
// batch per wave and at most the row kernels' count, which sizes the
// workspace.  bwd_pack = 1 keeps the row kernels; 4..32 forces S.
nr_status_t plan_bwd_packed(nr_dtype_t dt, int64_t rows, int64_t n, bool aligned, BwdPlan* pl,
                            int* S_out) {
  *S_out = 0;
  const int64_t nchunk = n / vec_elems(dt);
  if (!aligned || nchunk > 32 || tune(BWD_PACK) == 1) return NR_OK;
  int S = 4;
  while (S < nchunk) S *= 2;
  if (tune(BWD_PACK) > 1) S = tune(BWD_PACK);
  if ((S != 4 && S != 8 && S != 16 && S != 32) || S < nchunk) return NR_ERR_SHAPE;
  // at most five workgroups per CU (what ~100 VGPRs a lane leave resident),
  // the batches spread evenly over the rounds of the waves: 65536 x 256 bf16
  // RMSNorm 23.7 -> 21.2 us against 2048 workgroups of one batch a wave;
  // level (within 3%) at 655360..2621440 rows of 128 and 256
  const int64_t rw = nr::bwd_packed_rows_per_wave(S);
  const int64_t nb = (rows + rw - 1) / rw;
  const int64_t cap = pl->P < 1280 ? pl->P : 1280;
  const int64_t rounds = (nb + 4 * cap - 1) / (4 * cap);
  int64_t P = (nb + 4 * rounds - 1) / (4 * rounds);
  if (P > pl->P) P = pl->P;
  if (P < 1) P = 1;
  pl->P = static_cast<int>(P);
  *S_out = S;
  return NR_OK;
}

// Resident workgroups per CU wanted for a backward whose row takes W waves
// (about ten waves a CU, at most four workgroups).
// Rows of at most half a wave's chunks (16-bit rows of up to 256 elements,
// e.g. a per-head norm) take up to eight (65536 x 256 bf16 RMSNorm: 31.6 ->
// 25.7 us; 2621440 x 128: 889 -> 618 us).
int narrow_per_cu(int64_t W, int64_t nchunk) {
  if (W >= 6) return 1;
  if (nchunk <= 32) return 8;
  const int64_t k = 10 / W;
  return static_cast<int>(k > 4 ? 4 : k);
}

// Backward launch shape.
//   K, W: as few chunks per lane as lets at most 16 waves cover the row
//     (5120 bf16: K = 1, W = 10).
//   D (rows per batch) and PF (batches loaded ahead): by default the
//     largest that fit the 128-VGPR budget of a 1024-thread workgroup
//     without spilling (RMSNorm with one chunk per lane: D = 2 on aligned
//     rows, PF = 2; LayerNorm, which also carries the dbeta accumulators:
//     D = 1, PF = 1), and the measured shapes below for the rows of 5120
//     bf16 the workloads use.
//   P (workgroups): each handles about rows/P rows, dealt out round robin.
//     At least 8 rows per workgroup keep the fp32 partial rows small next
//     to the row traffic (under 9% extra at 16-bit storage, under 2% once
//     the cap below applies: 65536 rows).  Short batches want every CU busy
//     more than they want fewer partial rows: 3840 rows of 5120 bf16 took
//     25 us on 256 workgroups against 28 us on 240.  At most 256, or 512
//     where two workgroups of the shape fit a CU (LayerNorm and the fused
//     RMSNorm + RoPE with one or two batches ahead): on MI355X's 256 CUs
//     one or two resident workgroups per CU; more gave a second, partial
//     round of workgroups and measured slower.
//   Narrow rows, whose row takes few waves, leave a CU with little in flight
//   at one or two workgroups: there the cap is 256 times narrow_per_cu
//   (LayerNorm from 5 waves a row down, RMSNorm from 4; 15360 rows of bf16:
//   LayerNorm 2560 wide 72 -> 50 us on 512 workgroups, 1280 wide 56 -> 32 us
//   on 768, RMSNorm 1280 wide 38 -> 26 us on 768; RMSNorm 2560 wide measured
//   7% faster on 512 at 15360 rows but 4% slower at 65536, and keeps 256).
//   P depends on the shape (row count, width, element size) and the operator
//   only, so the summation order and the workspace size are the same on every
//   device.
void bwd_grid(int64_t rows, int per_cu, int64_t* P_out, int64_t* rpb_out,
              int64_t rows_min_default = 8) {
  const int64_t rows_min = tune(BWD_ROWS_MIN) > 0 ? tune(BWD_ROWS_MIN) : rows_min_default;
  const int64_t pcap = tune(BWD_P) > 0 ? tune(BWD_P) : 256 * static_cast<int64_t>(per_cu);
  int64_t P = tune(BWD_P) > 0 ? pcap : (rows + rows_min - 1) / rows_min;
  if (P > pcap) P = pcap;
  if (P > rows) P = rows;
  if (P < 1) P = 1;
  const int64_t rpb = rows > 0 ? (rows + P - 1) / P : 1;
  *P_out = rows > 0 ? (rows + rpb - 1) / rpb : 1;  // no empty workgroups
  *rpb_out = rpb;
}

nr_status_t plan_bwd(nr_dtype_t dt, bool ln, int64_t rows, int64_t n, bool aligned, BwdPlan* pl,
                     bool rope = false, bool gelu = false) {
  const int E = vec_elems(dt);
  const int64_t nchunk = (n + E - 1) / E;
  const int64_t need = (nchunk + 63) / 64;
  int K = 0, W = 0;
  for (int k : kBwdK) {
    if ((need + k - 1) / k <= 16) {
      K = k;
      break;
    }
  }
  if (tune(BWD_K) > 0) K = tune(BWD_K);
  if (K > 0) W = static_cast<int>((need + K - 1) / K);
  if (tune(BWD_W) > 0) W = tune(BWD_W);
  // (the fused RMSNorm + RoPE backward also holds each chunk's cos/sin: one
  // row per batch, two batches ahead.  Misaligned rows take the element-wise
  // path, whose two-row batch spilled: one row there, 1.5x faster at
  // 15360 x 5118 bf16)
  int D = (!ln && !rope && K == 1 && aligned) ? 2 : 1;
  int PF = ((!ln || gelu) && K == 1) ? 2 : 1;
  // LayerNorm (with or without GeLU), and the fused RMSNorm + RoPE
  // backward, on rows of one chunk per lane and at most 10 waves: one
  // workgroup per CU with three batches in flight (65536 x 5120 bf16:
  // LayerNorm 347 -> 333 us against two workgroups per CU with one batch
  // each, RMSNorm + RoPE 343 -> 336 us against two per CU with two batches
  // each; 15360 x 5120 bf16 LayerNorm + GeLU 116.8 -> 113.9 us against two
  // batches ahead, 146 us with two workgroups per CU)
  if ((ln || rope) && K == 1 && (need + K - 1) / K <= 10) PF = 3;
  // Plain RMSNorm on aligned rows of 8..10 chunk slots (4096..5120 bf16):
  //   batches of 16384 rows or more: two chunks per lane on half the waves
  //     (5120 bf16: 5 waves), one row per batch, two batches ahead -- fewer
  //     waves with more loads each; 65536 x 5120 bf16: 338 -> 329 us
  //     (5.96 -> 6.11 TB/s, two runs on different boxes);
  //   smaller batches: one row per batch, four batches ahead (3840 x 5120
  //     bf16: 26.6 -> 25.1 us).
  if (!ln && !rope && !gelu && aligned && K == 1 && need >= 8 && need <= 10 &&
      tune(BWD_K) == 0 && tune(BWD_W) == 0) {
    if (rows >= 16384) {
      K = 2;
      W = static_cast<int>((need + 1) / 2);
      D = 1;
      PF = 2;
    } else {
      D = 1;
      PF = 4;
    }
  }
  if (tune(BWD_D) > 0) D = tune(BWD_D);
  if (tune(BWD_PF) > 0) PF = tune(BWD_PF);
  if (!in_set(K, kBwdK, 4) || !in_set(D, kBwdD, 4) || K * D > 8 || W < 1 || W > 16)
    return NR_ERR_SHAPE;
  // deeper prefetch (3 or 4 batches) only for one chunk per lane, at most 2
  // rows per batch and 10 waves (one workgroup per CU)
  if (PF < 1 || PF > 4 || (PF > 2 && (K != 1 || D > 2 || W > 10))) return NR_ERR_SHAPE;
  if (static_cast<int64_t>(64) * W * K < nchunk) return NR_ERR_SHAPE;
  // two resident workgroups per CU only when two of them fit: 2 W waves
  // over the CU's 4 SIMDs at the kernels' ~76-100 VGPRs allow W <= 10
  // Plain RMSNorm on aligned 16-bit rows of 16385..32768 elements (32
  // elements a lane, up to 16 waves): one pass, dW accumulated in LDS, one
  // batch ahead.  Against the two passes (bf16): 4096 x 32768 222 -> 149 us
  // (5.4 TB/s), 16384 x 32768 852 -> 584 us, 4096 x 20480 148 -> 96 us,
  // 8192 x 16392 267 -> 154 us; 256 x 32768 level.
  const bool lacc = !ln && !rope && !gelu && aligned && E == 8 && n >= nr::kLongRowMin &&
                    n <= nr::kRmsOnePassMax;
  if (lacc) {
    if (K * E != 32 || W > 16) return NR_ERR_SHAPE;
    D = 1;
    PF = 1;
  }
  // (its rows are 32-64 KiB: one row per workgroup at least, where short
  // rows take eight; 256 x 32768 bf16: 40.9 us on 32 workgroups of 8 rows)
  int64_t P, rpb;
  int per_cu = (((ln && !gelu) || rope) && W <= 10 && PF <= 2) ? 2 : 1;
  if (!rope && !lacc && K == 1 && (ln ? W <= 5 : W <= 4)) {
    const int nw = narrow_per_cu(W, nchunk);
    if (nw > per_cu) per_cu = nw;
  }
  // RoPE rows of at most 32 16-bit chunks (a per-head q/k norm): up to five
  // a CU, as the packed backward of the plain norms takes (65536 tokens x 40
  // heads x 128 bf16: 450 -> 348 us against 512 workgroups)
  if (rope && (n + 7) / 8 <= 32) per_cu = 5;
  bwd_grid(rows, per_cu, &P, &rpb, lacc ? 1 : 8);
  *pl = BwdPlan{W, K, D, static_cast<int>(P), PF, rpb, aligned, lacc};
  return NR_OK;
}

// The in-place RoPE kernel updates every (batch, token, head) vector from
// one lane, so distinct vectors must not share an element.  Sufficient test
// (the usual one for strided views): order the axes of size > 1 by stride;
// each stride must reach past the whole block spanned by the axes inside it,
// starting from one head_dim-long vector.  A stride of 0 on such an axis
// (a broadcast view) fails it; transposed layouts such as [B, H, T, D] pass.
bool rope_vectors_disjoint(int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                           int64_t sb, int64_t st, int64_t sh) {
  int64_t size[3] = {heads, tokens, batch}, stride[3] = {sh, st, sb};
  int order[3] = {0, 1, 2};
  std::sort(order, order + 3, [&](int a, int b) { return stride[a] < stride[b]; });
  int64_t span = head_dim;  // elements covered by the axes handled so far
  for (int i : order) {
    if (size[i] <= 1) continue;
    if (stride[i] < span) return false;
    const int64_t extra = size[i] - 1;
    span = (extra > (INT64_MAX - span) / stride[i]) ? INT64_MAX : extra * stride[i] + span;
  }
  return true;
}

nr_status_t plan_rope(nr_dtype_t dt, int64_t heads, int64_t head_dim, bool aligned,
                      int64_t vectors, RopePlan* pl) {
  const int E = aligned ? vec_elems(dt) : 2;
  const int64_t cph = head_dim / E;
  const int64_t nchunk = heads * cph;
  // A token's chunks are shared by `groups` waves of about 4 chunks per
  // lane each (a 40 x 128 bf16 token: 640 chunks, 3 waves of 4): against
  // one wave of 10 chunks per token that measured 6.3 -> 6.45-6.5 TB/s on
  // 65536 such tokens and 6.0 -> 6.4 TB/s on 15360, i.e. the streaming-copy
  // ceiling.  Batches of fewer than 32768 token vectors take about 2
  // chunks per lane on more waves (40 x 128 bf16: 5 waves of 2; 15360
  // tokens 50.2 -> 49.3 us; at 65536 tokens the 4-chunk shape stays ahead).
  // Very long tokens keep at most 64 waves and loop.
  const int64_t per_wave = vectors < 32768 ? 128 : 256;
  int groups = static_cast<int>(std::min<int64_t>((nchunk + per_wave - 1) / per_wave, 64));
  if (tune(ROPE_GROUPS) > 0) groups = tune(ROPE_GROUPS);
  int K = pick_at_least((nchunk + 64 * groups - 1) / (64 * groups), kRopeK, 7);
  if (K == 0) K = 10;  // several passes over the heads
  if (tune(ROPE_K) > 0) K = tune(ROPE_K);
  int wpb = tune(ROPE_WPB) > 0 ? tune(ROPE_WPB) : 4;
  if (!in_set(K, kRopeK, 7) || wpb < 1 || wpb > 4) return NR_ERR_SHAPE;
  if (groups < 1 || groups > 64) return NR_ERR_SHAPE;
  *pl = RopePlan{K, wpb, groups, aligned, (64 % cph) == 0};
  return NR_OK;
}

}  // namespace

namespace nr {
int record_hip_error(hipError_t e) { return static_cast<int>(hip_status(e)); }
}  // namespace nr

extern "C" {

int64_t nr_norm_n_max(nr_dtype_t dt) {
  return kMaxChunksPerRow * (dt == NR_F32 ? 4 : 8);
}

const char* nr_status_str(nr_status_t s) {
  switch (s) {
    case NR_OK: return "ok";
    case NR_ERR_NULLPTR: return "required pointer is NULL";
    case NR_ERR_SHAPE: return "invalid shape or launch shape";
    case NR_ERR_DTYPE: return "unsupported dtype";
    case NR_ERR_UNSUPPORTED_N: return "row length beyond the supported maximum";
    case NR_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case NR_ERR_HIP: return "HIP launch failed";
    case NR_ERR_ALIAS: return "output partially overlaps an input";
    case NR_ERR_TUNE: return "unknown tuning key or value";
    default: break;
  }
  return "unknown status";
}

int nr_last_hip_error(void) { return t_last_hip; }

nr_status_t nr_tune(const char* key, int value) {
  if (key == nullptr || value < 0) return NR_ERR_TUNE;
  for (int i = 0; i < NKEYS; ++i) {
    if (std::strcmp(key, kTuneNames[i]) == 0) {
      g_tune[i].store(value, std::memory_order_relaxed);
      return NR_OK;
    }
  }
  return NR_ERR_TUNE;
}

size_t nr_bwd_workspace_bytes(int64_t rows, int64_t n, int op) {
  if (rows <= 0 || n < 1 || op < 0 || op > 2) return 0;
  int64_t P, rpb;
  // the most workgroups any dtype can take: 16-bit rows have the fewest
  // waves (one 8-element chunk a lane), so the most workgroups per CU
  int per_cu = op != 0 ? 2 : 1;
  const int64_t w16 = ((n + 7) / 8 + 63) / 64;
  if (op != 2 && (op == 1 ? w16 <= 5 : w16 <= 4)) {
    const int nw = narrow_per_cu(w16, (n + 7) / 8);
    if (nw > per_cu) per_cu = nw;
  }
  if (op == 2 && (n + 7) / 8 <= 32) per_cu = 5;
  bwd_grid(rows, per_cu, &P, &rpb, op == 0 && n >= nr::kLongRowMin ? 1 : 8);
  const size_t one_pass =
      static_cast<size_t>(P) * static_cast<size_t>(n) * sizeof(float) * (op == 1 ? 2u : 1u);
  if (nr::bwd_two_pass(op == 0, n)) {  // partial rows, then two fp32 terms per row
    // sized for 2-byte elements, whose shorter rows give the largest P
    const int64_t PL = nr::long_bwd_groups(rows, n, 2);
    return static_cast<size_t>(PL) * static_cast<size_t>(n) * sizeof(float) * (op == 1 ? 2u : 1u) +
           static_cast<size_t>(rows) * 2u * sizeof(float);
  }
  if (n < nr::kLongRowMin) return one_pass;
  // plain RMSNorm of 16385..32768 elements: one pass for aligned 16-bit
  // rows, two for the others; the larger of the two sizes
  const int64_t PL = nr::long_bwd_groups(rows, n, 2);
  const size_t two_pass = static_cast<size_t>(PL) * static_cast<size_t>(n) * sizeof(float) +
                          static_cast<size_t>(rows) * 2u * sizeof(float);
  return one_pass > two_pass ? one_pass : two_pass;
}

nr_status_t rmsnorm_fwd(nr_dtype_t dt, const void* x, const void* w, void* y, float* inv_rms,
                        int64_t rows, int64_t n, float eps, int gemma_offset, void* stream) {
  nr_status_t s;
  if ((s = check_dtype(dt)) != NR_OK) return s;
  if ((s = check_norm_shape(dt, rows, n)) != NR_OK) return s;
  if (rows == 0) return NR_OK;
  if (x == nullptr || y == nullptr) return NR_ERR_NULLPTR;
  const size_t bytes = static_cast<size_t>(rows * n) * elem_bytes(dt);
  if (bad_overlap(y, bytes, x, bytes)) return NR_ERR_ALIAS;
  if (!fwd_buffers_disjoint(dt, rows, n, x, w, nullptr, y, inv_rms, nullptr)) return NR_ERR_ALIAS;
  const bool aligned = (n % vec_elems(dt)) == 0 && aligned16(x) && aligned16(y) &&
                       (w == nullptr || aligned16(w));
  FwdPlan pl;
  if ((s = plan_fwd(dt, rows, n, aligned, &pl, kFwdRms)) != NR_OK) return s;
  if (!fwd_grid_ok(rows, pl)) return NR_ERR_SHAPE;
  return hip_status(nr::launch_norm_fwd(false, dt, pl, x, w, nullptr, y, inv_rms, nullptr, rows,
                                        static_cast<int>(n), eps, gemma_offset ? 1.0f : 0.0f,
                                        static_cast<hipStream_t>(stream)));
}

nr_status_t layernorm_fwd(nr_dtype_t dt, const void* x, const void* gamma, const void* beta,
                          void* y, float* mean, float* rstd, int64_t rows, int64_t n, float eps,
                          void* stream) {
  nr_status_t s;
  if ((s = check_dtype(dt)) != NR_OK) return s;
  if ((s = check_norm_shape(dt, rows, n)) != NR_OK) return s;
  if (rows == 0) return NR_OK;
  if (x == nullptr || y == nullptr) return NR_ERR_NULLPTR;
  const size_t bytes = static_cast<size_t>(rows * n) * elem_bytes(dt);
  if (bad_overlap(y, bytes, x, bytes)) return NR_ERR_ALIAS;
  if (!fwd_buffers_disjoint(dt, rows, n, x, gamma, beta, y, mean, rstd)) return NR_ERR_ALIAS;
  const bool aligned = (n % vec_elems(dt)) == 0 && aligned16(x) && aligned16(y) &&
                       (gamma == nullptr || aligned16(gamma)) &&
                       (beta == nullptr || aligned16(beta));
  FwdPlan pl;
  if ((s = plan_fwd(dt, rows, n, aligned, &pl, kFwdLn)) != NR_OK) return s;
  if (!fwd_grid_ok(rows, pl)) return NR_ERR_SHAPE;
  return hip_status(nr::launch_norm_fwd(true, dt, pl, x, gamma, beta, y, mean, rstd, rows,
                                        static_cast<int>(n), eps, 0.0f,
                                        static_cast<hipStream_t>(stream)));
}

namespace {

// Backward of rows of kLongRowMin or more elements: pass A stores two fp32
// terms per row after the partial rows in the workspace, pass B writes dx
// and the partial rows, stage 2 adds those.
nr_status_t bwd_long(nr_dtype_t dt, bool ln, int epi, bool aligned, const void* dy, const void* x,
                     const void* w, const void* beta, const float* mean, const float* rstat,
                     void* dx, float* o0, float* o1, int64_t rows, int64_t n, float w_add,
                     const nr::RopeArgs& ra, void* workspace, size_t workspace_bytes,
                     hipStream_t st) {
  if (rows > INT32_MAX) return NR_ERR_SHAPE;  // pass A: one workgroup per row
  const bool want_cols = o0 != nullptr || o1 != nullptr;
  const int64_t P = nr::long_bwd_groups(rows, n, dt == NR_F32 ? 4 : 2);
  const size_t part_bytes =
      want_cols ? static_cast<size_t>(P) * n * sizeof(float) * (ln ? 2u : 1u) : 0u;
  const size_t need = part_bytes + static_cast<size_t>(rows) * 2u * sizeof(float);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
    return NR_ERR_WORKSPACE;
  float* part = want_cols ? static_cast<float*>(workspace) : nullptr;
  float* terms = reinterpret_cast<float*>(static_cast<char*>(workspace) + part_bytes);
  nr_status_t s = hip_status(nr::launch_norm_bwd_long(dt, ln, epi, aligned, dy, x, w, beta, mean,
                                                      rstat, terms, dx, part, P, rows,
                                                      static_cast<int>(n), w_add, ra, st));
  if (s != NR_OK || !want_cols) return s;
  // at most 51 partial rows, n/64 >= 256 column workgroups: about four
  // partial rows per slice (16 slices of one row each measured 8 us for the
  // 8 MB of a 65536-wide LayerNorm, 4 slices 4.7 us)
  const int slices = static_cast<int>(P >= 64 ? 16 : (P + 3) / 4);
  return hip_status(nr::launch_colreduce(part, P * n, static_cast<int>(P), static_cast<int>(n), o0,
                                         o1, st, slices < 1 ? 1 : slices));
}

nr_status_t norm_bwd_common(bool ln, nr_dtype_t dt, const void* dy, const void* x, const void* w,
                            const float* mean, const float* rstat, void* dx, float* o0, float* o1,
                            int64_t rows, int64_t n, float w_add, void* workspace,
                            size_t workspace_bytes, void* stream, bool gelu = false,
                            const void* beta = nullptr) {
  nr_status_t s;
  if ((s = check_dtype(dt)) != NR_OK) return s;
  if ((s = check_norm_shape(dt, rows, n)) != NR_OK) return s;
  const bool want_cols = o0 != nullptr || o1 != nullptr;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (rows == 0) {
    // empty batch: the column gradients are sums over no rows.  The column
    // reduction over zero partials writes the zeros (a kernel, not a memset,
    // so the call stays safe to record into a graph).
    if (!want_cols) return NR_OK;
    return hip_status(
        nr::launch_colreduce(nullptr, 0, 0, static_cast<int>(n), o0, o1, st));
  }
  if (dy == nullptr || x == nullptr || dx == nullptr || rstat == nullptr ||
      (ln && mean == nullptr))
    return NR_ERR_NULLPTR;
  const size_t bytes = static_cast<size_t>(rows * n) * elem_bytes(dt);
  if (bad_overlap(dx, bytes, dy, bytes) || bad_overlap(dx, bytes, x, bytes)) return NR_ERR_ALIAS;
  if (!bwd_buffers_disjoint(dt, rows, n, dy, x, w, beta, mean, rstat, dx, o0, o1, workspace,
                            workspace_bytes))
    return NR_ERR_ALIAS;
  const bool aligned = (n % vec_elems(dt)) == 0 && aligned16(dy) && aligned16(x) &&
                       aligned16(dx) && (w == nullptr || aligned16(w)) &&
                       (beta == nullptr || aligned16(beta));
  if (nr::bwd_two_pass(!ln && !gelu && aligned && vec_elems(dt) == 8, n)) {
    const nr::RopeArgs none{nullptr, nullptr, 2, 1};
    return bwd_long(dt, ln, gelu ? 2 : 0, aligned, dy, x, w, beta, mean, rstat, dx, o0, o1, rows,
                    n, w_add, none, workspace, workspace_bytes, st);
  }
  BwdPlan pl;
  if ((s = plan_bwd(dt, ln, rows, n, aligned, &pl, false, gelu)) != NR_OK) return s;
  // LayerNorm + GeLU on 16-bit rows of 2560 or 5120: 10 elements a lane on
  // n / 640 waves, which load the CU's four SIMDs evenly (the one-chunk
  // layout puts 10 waves on them 3/3/2/2).  The 4-wave form (2560) takes two
  // workgroups per CU once the batch gives each one 16 rows (15360 x 2560
  // bf16: 63 -> 51 us against one per CU; at 3840 rows, 8 rows each, 23 -> 26
  // us); the 8-wave form keeps the usual count (95 against 93 us with two)
  int S = 0;
  if ((s = plan_bwd_packed(dt, rows, n, aligned, &pl, &S)) != NR_OK) return s;
  const bool pair = gelu && nr::ln_gelu_pair_fits(dt, n, aligned);
  if (pair && n / 640 == 4) {
    int64_t P2, rpb2;
    bwd_grid(rows, 2, &P2, &rpb2, 16);
    pl.P = static_cast<int>(P2);
  }
  float* part = nullptr;
  if (want_cols) {
    const size_t need = static_cast<size_t>(pl.P) * n * sizeof(float) * (ln ? 2 : 1);
    if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
      return NR_ERR_WORKSPACE;
    part = static_cast<float*>(workspace);
  }
  const nr::RopeArgs none{nullptr, nullptr, 2, 1};
  const hipError_t e =
      S > 0 ? nr::launch_bwd_packed(dt, ln, gelu ? 2 : 0, S, pl.P, dy, x, w,
                                    beta, mean, rstat, dx, part, rows, static_cast<int>(n), w_add,
                                    none, st)
      : pair ? nr::launch_ln_gelu_bwd_pair(dt, pl.P, dy, x, w, beta, mean, rstat, dx, part, rows,
                                         static_cast<int>(n), st)
      : gelu ? nr::launch_ln_gelu_bwd(dt, pl, dy, x, w, beta, mean, rstat, dx, part, rows,
                                      static_cast<int>(n), st)
             : nr::launch_norm_bwd(ln, dt, pl, dy, x, w, mean, rstat, dx, part, rows,
                                   static_cast<int>(n), w_add, st);
  if ((s = hip_status(e)) != NR_OK) return s;
  if (want_cols)
    return hip_status(nr::launch_colreduce(part, static_cast<int64_t>(pl.P) * n, pl.P,
                                           static_cast<int>(n), o0, o1, st));
  return NR_OK;
}

}  // namespace

nr_status_t rmsnorm_bwd(nr_dtype_t dt, const void* dy, const void* x, const void* w,
                        const float* inv_rms, void* dx, float* dw, int64_t rows, int64_t n,
                        int gemma_offset, void* workspace, size_t workspace_bytes, void* stream) {
  return norm_bwd_common(false, dt, dy, x, w, nullptr, inv_rms, dx, dw, nullptr, rows, n,
                         gemma_offset ? 1.0f : 0.0f, workspace, workspace_bytes, stream);
}

nr_status_t layernorm_bwd(nr_dtype_t dt, const void* dy, const void* x, const void* gamma,
                          const float* mean, const float* rstd, void* dx, float* dgamma,
                          float* dbeta, int64_t rows, int64_t n, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return norm_bwd_common(true, dt, dy, x, gamma, mean, rstd, dx, dgamma, dbeta, rows, n, 0.0f,
                         workspace, workspace_bytes, stream);
}

nr_status_t layernorm_gelu_fwd(nr_dtype_t dt, const void* x, const void* gamma, const void* beta,
                               void* y, float* mean, float* rstd, int64_t rows, int64_t n,
                               float eps, void* stream) {
  nr_status_t s;
  if ((s = check_dtype(dt)) != NR_OK) return s;
  if ((s = check_norm_shape(dt, rows, n)) != NR_OK) return s;
  if (rows == 0) return NR_OK;
  if (x == nullptr || y == nullptr) return NR_ERR_NULLPTR;
  const size_t bytes = static_cast<size_t>(rows * n) * elem_bytes(dt);
  if (bad_overlap(y, bytes, x, bytes)) return NR_ERR_ALIAS;
  if (!fwd_buffers_disjoint(dt, rows, n, x, gamma, beta, y, mean, rstd)) return NR_ERR_ALIAS;
  const bool aligned = (n % vec_elems(dt)) == 0 && aligned16(x) && aligned16(y) &&
                       (gamma == nullptr || aligned16(gamma)) &&
                       (beta == nullptr || aligned16(beta));
  FwdPlan pl;
  if ((s = plan_fwd(dt, rows, n, aligned, &pl, kFwdLn)) != NR_OK) return s;
  if (!fwd_grid_ok(rows, pl)) return NR_ERR_SHAPE;
  return hip_status(nr::launch_ln_gelu_fwd(dt, pl, x, gamma, beta, y, mean, rstd, rows,
                                           static_cast<int>(n), eps,
                                           static_cast<hipStream_t>(stream)));
}

nr_status_t layernorm_gelu_bwd(nr_dtype_t dt, const void* dout, const void* x, const void* gamma,
                               const void* beta, const float* mean, const float* rstd, void* dx,
                               float* dgamma, float* dbeta, int64_t rows, int64_t n,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return norm_bwd_common(true, dt, dout, x, gamma, mean, rstd, dx, dgamma, dbeta, rows, n, 0.0f,
                         workspace, workspace_bytes, stream, true, beta);
}

namespace {

// Checks shared by the fused RMSNorm + RoPE calls: whole heads per row, an
// even head size, a token index per row; reports whether the 128-bit path
// applies to the tables.
nr_status_t check_rope_rows(nr_dtype_t dt, const float* cos_tab, const float* sin_tab,
                            int64_t n, int64_t head_dim, int64_t rows_per_token, bool* vec_ok) {
  if (head_dim < 2 || (head_dim & 1) || n % head_dim != 0 || rows_per_token < 1)
    return NR_ERR_SHAPE;
  if (cos_tab == nullptr || sin_tab == nullptr) return NR_ERR_NULLPTR;
  *vec_ok = head_dim % vec_elems(dt) == 0 && aligned16(cos_tab) && aligned16(sin_tab);
  return NR_OK;
}

}  // namespace

nr_status_t rmsnorm_rope_fwd(nr_dtype_t dt, const void* x, const void* w, void* y, float* inv_rms,
                             const float* cos_tab, const float* sin_tab, int64_t rows, int64_t n,
                             int64_t head_dim, int64_t rows_per_token, float eps,
                             int gemma_offset, void* stream) {
  nr_status_t s;
  if ((s = check_dtype(dt)) != NR_OK) return s;
  if ((s = check_norm_shape(dt, rows, n)) != NR_OK) return s;
  if (head_dim < 2 || (head_dim & 1) || n % head_dim != 0 || rows_per_token < 1)
    return NR_ERR_SHAPE;
  if (rows == 0) return NR_OK;
  if (x == nullptr || y == nullptr) return NR_ERR_NULLPTR;
  bool vec_tab;
  if ((s = check_rope_rows(dt, cos_tab, sin_tab, n, head_dim, rows_per_token, &vec_tab)) != NR_OK)
    return s;
  const size_t bytes = static_cast<size_t>(rows * n) * elem_bytes(dt);
  if (bad_overlap(y, bytes, x, bytes)) return NR_ERR_ALIAS;
  const size_t tab_bytes =
      static_cast<size_t>((rows + rows_per_token - 1) / rows_per_token) * (head_dim / 2) * 4;
  if (!fwd_buffers_disjoint(dt, rows, n, x, w, nullptr, y, inv_rms, nullptr, cos_tab, sin_tab,
                            tab_bytes))
    return NR_ERR_ALIAS;
  const bool aligned = vec_tab && (n % vec_elems(dt)) == 0 && aligned16(x) && aligned16(y) &&
                       (w == nullptr || aligned16(w));
  FwdPlan pl;
  if ((s = plan_fwd(dt, rows, n, aligned, &pl, kFwdRmsRope)) != NR_OK) return s;
  if (!fwd_grid_ok(rows, pl)) return NR_ERR_SHAPE;
  const nr::RopeArgs ra{cos_tab, sin_tab, static_cast<int>(head_dim), rows_per_token};
  return hip_status(nr::launch_rms_rope_fwd(dt, pl, x, w, y, inv_rms, ra, rows, static_cast<int>(n),
                                            eps, gemma_offset ? 1.0f : 0.0f,
                                            static_cast<hipStream_t>(stream)));
}

nr_status_t rmsnorm_rope_bwd(nr_dtype_t dt, const void* dout, const void* x, const void* w,
                             const float* inv_rms, const float* cos_tab, const float* sin_tab,
                             void* dx, float* dw, int64_t rows, int64_t n, int64_t head_dim,
                             int64_t rows_per_token, int gemma_offset, void* workspace,
                             size_t workspace_bytes, void* stream) {
  nr_status_t s;
  if ((s = check_dtype(dt)) != NR_OK) return s;
  if ((s = check_norm_shape(dt, rows, n)) != NR_OK) return s;
  if (head_dim < 2 || (head_dim & 1) || n % head_dim != 0 || rows_per_token < 1)
    return NR_ERR_SHAPE;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (rows == 0) {
    if (dw == nullptr) return NR_OK;
    return hip_status(
        nr::launch_colreduce(nullptr, 0, 0, static_cast<int>(n), dw, nullptr, st));
  }
  if (dout == nullptr || x == nullptr || dx == nullptr || inv_rms == nullptr) return NR_ERR_NULLPTR;
  bool vec_tab;
  if ((s = check_rope_rows(dt, cos_tab, sin_tab, n, head_dim, rows_per_token, &vec_tab)) != NR_OK)
    return s;
  const size_t bytes = static_cast<size_t>(rows * n) * elem_bytes(dt);
  if (bad_overlap(dx, bytes, dout, bytes) || bad_overlap(dx, bytes, x, bytes)) return NR_ERR_ALIAS;
  // the tables: head_dim / 2 angles per token
  const size_t tab_bytes =
      static_cast<size_t>((rows + rows_per_token - 1) / rows_per_token) * (head_dim / 2) * 4;
  if (!bwd_buffers_disjoint(dt, rows, n, dout, x, w, nullptr, nullptr, inv_rms, dx, dw, nullptr,
                            workspace, workspace_bytes, cos_tab, sin_tab, tab_bytes))
    return NR_ERR_ALIAS;
  const bool aligned = vec_tab && (n % vec_elems(dt)) == 0 && aligned16(dout) && aligned16(x) &&
                       aligned16(dx) && (w == nullptr || aligned16(w));
  const nr::RopeArgs ra{cos_tab, sin_tab, static_cast<int>(head_dim), rows_per_token};
  if (nr::bwd_two_pass(false, n))
    return bwd_long(dt, false, 1, aligned, dout, x, w, nullptr, nullptr, inv_rms, dx, dw, nullptr,
                    rows, n, gemma_offset ? 1.0f : 0.0f, ra, workspace, workspace_bytes, st);
  BwdPlan pl;
  if ((s = plan_bwd(dt, false, rows, n, aligned, &pl, true)) != NR_OK) return s;
  int S = 0;
  if ((s = plan_bwd_packed(dt, rows, n, aligned, &pl, &S)) != NR_OK) return s;
  float* part = nullptr;
  if (dw != nullptr) {
    const size_t need = static_cast<size_t>(pl.P) * n * sizeof(float);
    if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
      return NR_ERR_WORKSPACE;
    part = static_cast<float*>(workspace);
  }
  if ((s = hip_status(
           S > 0 ? nr::launch_bwd_packed(dt, false, 1, S, pl.P, dout, x, w, nullptr,
                                         nullptr, inv_rms, dx, part, rows, static_cast<int>(n),
                                         gemma_offset ? 1.0f : 0.0f, ra, st)
                 : nr::launch_rms_rope_bwd(dt, pl, dout, x, w, inv_rms, ra, dx, part, rows,
                                           static_cast<int>(n), gemma_offset ? 1.0f : 0.0f,
                                           st))) != NR_OK)
    return s;
  if (dw != nullptr)
    return hip_status(nr::launch_colreduce(part, static_cast<int64_t>(pl.P) * n, pl.P,
                                           static_cast<int>(n), dw, nullptr, st));
  return NR_OK;
}

nr_status_t rope_interleaved_apply(nr_dtype_t dt, void* x, const float* cos_tab,
                                   const float* sin_tab, int64_t batch, int64_t tokens,
                                   int64_t heads, int64_t head_dim, int64_t stride_batch,
                                   int64_t stride_token, int64_t stride_head, int inverse,
                                   void* stream) {
  nr_status_t s;
  if ((s = check_dtype(dt)) != NR_OK) return s;
  if (batch < 0 || tokens < 0 || heads < 0 || head_dim < 2 || (head_dim & 1)) return NR_ERR_SHAPE;
  if (stride_batch < 0 || stride_token < 0 || stride_head < 0) return NR_ERR_SHAPE;
  if (heads > (int64_t{1} << 20) || head_dim > (int64_t{1} << 20) ||
      heads * head_dim > (int64_t{1} << 30))
    return NR_ERR_UNSUPPORTED_N;
  if (batch == 0 || tokens == 0 || heads == 0) return NR_OK;
  if (tokens > INT64_MAX / head_dim || batch > INT64_MAX / tokens) return NR_ERR_SHAPE;
  if (!rope_vectors_disjoint(batch, tokens, heads, head_dim, stride_batch, stride_token,
                             stride_head))
    return NR_ERR_ALIAS;
  if (x == nullptr || cos_tab == nullptr || sin_tab == nullptr) return NR_ERR_NULLPTR;
  // x is rewritten while the tables are read: its extent (saturating) may not
  // share a byte with either table (head_dim / 2 fp32 angles per token)
  {
    int64_t ext = head_dim;  // elements from x to one past its last element
    const int64_t cnt[3] = {batch - 1, tokens - 1, heads - 1};
    const int64_t str[3] = {stride_batch, stride_token, stride_head};
    for (int i = 0; i < 3; ++i) {
      if (str[i] > 0 && cnt[i] > (INT64_MAX - ext) / str[i]) ext = INT64_MAX;
      else if (ext != INT64_MAX) ext += cnt[i] * str[i];
    }
    const int64_t e = elem_bytes(dt);
    const size_t xb = ext > INT64_MAX / e ? SIZE_MAX : static_cast<size_t>(ext * e);
    const size_t tb = static_cast<size_t>(tokens) * static_cast<size_t>(head_dim / 2) * 4u;
    if (any_overlap(x, xb, cos_tab, tb) || any_overlap(x, xb, sin_tab, tb)) return NR_ERR_ALIAS;
  }
  // a token's heads are addressed with 32-bit byte offsets from the token start
  const int64_t span = ((heads - 1) * stride_head + head_dim) * elem_bytes(dt);
  if (stride_head > (int64_t{1} << 30) || span >= (int64_t{1} << 30)) return NR_ERR_UNSUPPORTED_N;
  const int v = vec_elems(dt);
  const bool aligned = head_dim % v == 0 && stride_batch % v == 0 && stride_token % v == 0 &&
                       stride_head % v == 0 && aligned16(x) && aligned16(cos_tab) &&
                       aligned16(sin_tab);
  RopePlan pl;
  if ((s = plan_rope(dt, heads, head_dim, aligned, batch * tokens, &pl)) != NR_OK) return s;
  // `groups` waves per token, waves_per_block waves per workgroup: the grid
  // must fit the hardware's 2^31 - 1 workgroups
  if (batch * tokens > INT64_MAX / 64 ||
      (batch * tokens * pl.groups + pl.waves_per_block - 1) / pl.waves_per_block > INT32_MAX)
    return NR_ERR_SHAPE;
  return hip_status(nr::launch_rope(dt, pl, x, cos_tab, sin_tab, batch, tokens,
                                    static_cast<int>(heads), static_cast<int>(head_dim),
                                    stride_batch, stride_token, stride_head,
                                    inverse ? -1.0f : 1.0f, static_cast<hipStream_t>(stream)));
}

nr_status_t rope_table_1d(float* cos_tab, float* sin_tab, int64_t tokens, int64_t head_dim,
                          int64_t pos0, double theta, void* stream) {
  if (tokens < 0 || head_dim < 2 || (head_dim & 1) || head_dim > (int64_t{1} << 20))
    return NR_ERR_SHAPE;
  if (!(theta > 0.0)) return NR_ERR_SHAPE;
  if (tokens == 0) return NR_OK;
  if (tokens > INT64_MAX / head_dim) return NR_ERR_SHAPE;
  if (cos_tab == nullptr || sin_tab == nullptr) return NR_ERR_NULLPTR;
  const size_t tb = static_cast<size_t>(tokens * (head_dim / 2)) * sizeof(float);
  if (any_overlap(cos_tab, tb, sin_tab, tb)) return NR_ERR_ALIAS;
  return hip_status(nr::launch_rope_table_1d(cos_tab, sin_tab, tokens, static_cast<int>(head_dim),
                                             pos0, theta, static_cast<hipStream_t>(stream)));
}

nr_status_t rope_table_3d(float* cos_tab, float* sin_tab, int64_t frames, int64_t height,
                          int64_t width, int64_t pairs_t, int64_t pairs_h, int64_t pairs_w,
                          double theta, void* stream) {
  if (frames < 0 || height < 0 || width < 0) return NR_ERR_SHAPE;
  if (pairs_t < 1 || pairs_h < 1 || pairs_w < 1 || pairs_t + pairs_h + pairs_w > (1 << 19))
    return NR_ERR_SHAPE;
  if (!(theta > 0.0)) return NR_ERR_SHAPE;
  if (frames == 0 || height == 0 || width == 0) return NR_OK;
  if (height > INT64_MAX / width || frames > INT64_MAX / (height * width) / (1 << 20))
    return NR_ERR_SHAPE;
  if (cos_tab == nullptr || sin_tab == nullptr) return NR_ERR_NULLPTR;
  const size_t tb =
      static_cast<size_t>(frames * height * width * (pairs_t + pairs_h + pairs_w)) * sizeof(float);
  if (any_overlap(cos_tab, tb, sin_tab, tb)) return NR_ERR_ALIAS;
  return hip_status(nr::launch_rope_table_3d(
      cos_tab, sin_tab, frames, height, width, static_cast<int>(pairs_t),
      static_cast<int>(pairs_h), static_cast<int>(pairs_w), theta,
      static_cast<hipStream_t>(stream)));
}

// Output tile of the RMSNorm -> linear kernels: 256 x 256 (direct-to-LDS,
// folded weight) whenever N allows it -- measured faster than the 128 x 128
// kernel at every M tried, from 1024 rows (80 tiles: 141 against 144 us) to
// 65536 (2.72 against 5.76 ms) at N = K = 5120 -- else 128 x 128.  The tuning
// table can force either.
namespace {
int linear_tile(int64_t /*M*/, int64_t N) {
  int tile = N % 256 == 0 ? 2 : 1;
  if (tune(GEMM_TILE) > 0) tile = tune(GEMM_TILE);
  return tile;
}
}  // namespace

size_t nr_rmsnorm_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int has_weight) {
  if (M <= 0 || M > INT32_MAX || N <= 0 || K <= 0 || N > (int64_t{1} << 22) || K > 65536) return 0;
  if (linear_tile(M, N) != 2) return 0;
  return nr::linear_rows_bytes(M) + (has_weight ? static_cast<size_t>(N * K) * 2 : 0);
}

nr_status_t rmsnorm_linear_fwd(nr_dtype_t dt, const void* x, const void* w_norm, const void* W,
                               void* out, float* inv_rms, int64_t M, int64_t N, int64_t K,
                               float eps, int gemma_offset, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (dt != NR_BF16) return NR_ERR_DTYPE;  // the bf16 matrix cores only
  if (M < 0 || M > INT32_MAX || N < 128 || N % 128 != 0 || K < 64 || K % 64 != 0)
    return NR_ERR_SHAPE;
  if (K > 65536 || N > (int64_t{1} << 22)) return NR_ERR_UNSUPPORTED_N;
  if (M == 0) return NR_OK;
  if (x == nullptr || W == nullptr || out == nullptr) return NR_ERR_NULLPTR;
  if (!aligned16(x) || !aligned16(W) || !aligned16(out) || (w_norm != nullptr && !aligned16(w_norm)))
    return NR_ERR_SHAPE;
  if (M > INT64_MAX / K / 2 || M > INT64_MAX / N / 2) return NR_ERR_SHAPE;
  const int tile = linear_tile(M, N);
  if (tile < 1 || tile > 2 || (tile == 2 && N % 256 != 0)) return NR_ERR_SHAPE;
  const int64_t edge = tile == 2 ? 256 : 128;
  if (((M + edge - 1) / edge) * (N / edge) > INT32_MAX) return NR_ERR_SHAPE;
  const size_t xb = static_cast<size_t>(M * K) * 2, wb = static_cast<size_t>(N * K) * 2,
               ob = static_cast<size_t>(M * N) * 2;
  if (bad_overlap(out, ob, x, xb) || out == x || bad_overlap(out, ob, W, wb) || out == W)
    return NR_ERR_ALIAS;
  if (tile == 2 && (w_norm != nullptr || inv_rms == nullptr)) {
    // the row statistics (unless inv_rms takes them), then the folded weight
    // (N K bf16): 16-byte aligned, apart from every operand
    const size_t need = nr::linear_rows_bytes(M) + (w_norm != nullptr ? wb : 0);
    if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
      return NR_ERR_WORKSPACE;
    const size_t rb = static_cast<size_t>(M) * 4;
    if (bad_overlap(workspace, need, x, xb) || bad_overlap(workspace, need, W, wb) ||
        bad_overlap(workspace, need, out, ob) ||
        bad_overlap(workspace, need, w_norm, static_cast<size_t>(K) * 2) ||
        bad_overlap(workspace, need, inv_rms, rb) || workspace == x || workspace == W ||
        workspace == out || workspace == w_norm || workspace == inv_rms)
      return NR_ERR_ALIAS;
  }
  return hip_status(nr::launch_rmsnorm_linear(x, w_norm, W, out, inv_rms, workspace,
                                              static_cast<int>(M), static_cast<int>(N),
                                              static_cast<int>(K), eps, gemma_offset ? 1.0f : 0.0f,
                                              tile, static_cast<hipStream_t>(stream)));
}

size_t nr_layernorm_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int has_gamma) {
  if (M <= 0 || M > INT32_MAX || N <= 0 || K <= 0 || N > (int64_t{1} << 22) || K > 65536) return 0;
  return nr::layernorm_linear_ws_bytes(M, N, K, has_gamma != 0);
}

nr_status_t layernorm_linear_fwd(nr_dtype_t dt, const void* x, const void* gamma, const void* beta,
                                 const void* W, void* out, float* mean, float* rstd, int64_t M,
                                 int64_t N, int64_t K, float eps, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (dt != NR_BF16) return NR_ERR_DTYPE;  // the bf16 matrix cores only
  if (M < 0 || M > INT32_MAX || N < 256 || N % 256 != 0 || K < 64 || K % 64 != 0)
    return NR_ERR_SHAPE;
  if (K > 65536 || N > (int64_t{1} << 22)) return NR_ERR_UNSUPPORTED_N;
  if (M == 0) return NR_OK;
  if (x == nullptr || W == nullptr || out == nullptr) return NR_ERR_NULLPTR;
  if (!aligned16(x) || !aligned16(W) || !aligned16(out) ||
      (gamma != nullptr && !aligned16(gamma)) || (beta != nullptr && !aligned16(beta)))
    return NR_ERR_SHAPE;
  if (M > INT64_MAX / K / 2 || M > INT64_MAX / N / 2) return NR_ERR_SHAPE;
  if (((M + 255) / 256) * (N / 256) > INT32_MAX) return NR_ERR_SHAPE;
  const size_t xb = static_cast<size_t>(M * K) * 2, wb = static_cast<size_t>(N * K) * 2,
               ob = static_cast<size_t>(M * N) * 2, rb = static_cast<size_t>(M) * 4,
               vb = static_cast<size_t>(K) * 2;
  if (bad_overlap(out, ob, x, xb) || out == x || bad_overlap(out, ob, W, wb) || out == W)
    return NR_ERR_ALIAS;
  const size_t need = nr::layernorm_linear_ws_bytes(M, N, K, gamma != nullptr);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
    return NR_ERR_WORKSPACE;
  const void* ops[] = {x, W, out, gamma, beta, mean, rstd};
  const size_t opb[] = {xb, wb, ob, vb, vb, rb, rb};
  for (int i = 0; i < 7; ++i)
    if (ops[i] == workspace || bad_overlap(workspace, need, ops[i], opb[i])) return NR_ERR_ALIAS;
  if (mean != nullptr && rstd != nullptr && (mean == rstd || bad_overlap(mean, rb, rstd, rb)))
    return NR_ERR_ALIAS;
  return hip_status(nr::launch_layernorm_linear(x, gamma, beta, W, out, mean, rstd, workspace,
                                                static_cast<int>(M), static_cast<int>(N),
                                                static_cast<int>(K), eps,
                                                static_cast<hipStream_t>(stream)));
}

nr_status_t rmsnorm_linear_fold_weight(nr_dtype_t dt, const void* w_norm, const void* W,
                                       void* W_folded, int64_t N, int64_t K, int gemma_offset,
                                       void* stream) {
  if (dt != NR_BF16) return NR_ERR_DTYPE;
  if (N < 0 || K < 0 || K % 8 != 0) return NR_ERR_SHAPE;
  if (K > 65536 || N > (int64_t{1} << 22)) return NR_ERR_UNSUPPORTED_N;
  if (N == 0 || K == 0) return NR_OK;
  if (w_norm == nullptr || W == nullptr || W_folded == nullptr) return NR_ERR_NULLPTR;
  if (!aligned16(w_norm) || !aligned16(W) || !aligned16(W_folded)) return NR_ERR_SHAPE;
  const size_t wb = static_cast<size_t>(N * K) * 2;
  // in place (W_folded == W) is fine: each element is read, then written, by one lane
  if ((bad_overlap(W_folded, wb, W, wb) && W_folded != W) ||
      bad_overlap(W_folded, wb, w_norm, static_cast<size_t>(K) * 2) || W_folded == w_norm)
    return NR_ERR_ALIAS;
  return hip_status(nr::launch_fold_norm_weight(w_norm, W, W_folded, N, static_cast<int>(K),
                                                gemma_offset ? 1.0f : 0.0f,
                                                static_cast<hipStream_t>(stream)));
}

nr_status_t nr_stream_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes == 0) return NR_OK;
  if (src == nullptr || dst == nullptr) return NR_ERR_NULLPTR;
  if ((bytes & 15u) != 0 || !aligned16(src) || !aligned16(dst)) return NR_ERR_SHAPE;
  const int64_t nvec = static_cast<int64_t>(bytes / 16);
  // one workgroup per 4 KiB: the grid must fit the hardware's 2^31 - 1
  if ((nvec + 255) / 256 > INT32_MAX) return NR_ERR_SHAPE;
  if (bad_overlap(dst, bytes, src, bytes) || dst == src) return NR_ERR_ALIAS;
  return hip_status(nr::launch_stream_copy(src, dst, nvec, static_cast<hipStream_t>(stream)));
}

nr_status_t nr_stream_mix(const void* a, const void* b, void* dst, size_t bytes, int write,
                          void* stream) {
  if (bytes == 0) return NR_OK;
  if (a == nullptr || b == nullptr || dst == nullptr) return NR_ERR_NULLPTR;
  if ((bytes & 15u) != 0 || !aligned16(a) || !aligned16(b) || !aligned16(dst)) return NR_ERR_SHAPE;
  const int64_t nvec = static_cast<int64_t>(bytes / 16);
  if ((nvec + 255) / 256 > INT32_MAX) return NR_ERR_SHAPE;
  if (bad_overlap(dst, bytes, a, bytes) || bad_overlap(dst, bytes, b, bytes) || dst == a ||
      dst == b)
    return NR_ERR_ALIAS;
  return hip_status(nr::launch_stream_mix(a, b, dst, nvec, write != 0,
                                          static_cast<hipStream_t>(stream)));
}

}  // extern "C"
