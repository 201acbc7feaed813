// Coarse stage of VSA: cube-level attention and the top-K block selection.
//
// Input: fp32 means of q, k, v per cube, [B,H,C,D] (written by the reorder).
// Two workgroups (16 waves each) own 16 query-cube rows of one head; both
// compute
//   1. Sc[16, C] = Qc Kc^T / sqrt(D) on fp32 MFMA (v_mfma_f32_16x16x4_f32),
//      kept in LDS (16 x C fp32, C <= 2048) and optionally written out;
// then the first one does
//   2. row max and 1/sum(exp) per row (one wave per row, wave reductions);
//   3. O_coarse[16, D] = softmax(Sc) Vc on fp32 MFMA, probabilities formed on
//      the fly from the LDS scores, each 16-wide slice of D split over waves
//      by key batches and summed through LDS (their first Vc loads are issued
//      at the start so that the latency overlaps phase 1);
// and the second one
//   4. the top-K of each row (one row per wave): the K-th largest score is
//      found exactly by a 32-step bitwise search over order-preserving uint32
//      keys of the fp32 scores, each step counting with 64-bit wave ballots
//      (no shuffles); then one ordered pass with ballots emits every index
//      above it plus the lowest-index ties, already in ascending order.
// The split costs one more score computation and lets the two phases run on
// separate CUs instead of competing for one CU's issue slots; it pays while
// the grid leaves CUs idle (small C).  For larger problems one workgroup runs
// both phases on one copy of the scores (grid z = 1).
// Everything is fp32 (no bf16 rounding of means or scores), so the selection
// differs from an exact one only where two scores are within fp32 rounding.
#include "vsa_internal.h"
#include "vsa_bwd.h"
#include "block_lists.h"

#include <algorithm>
#include <type_traits>

namespace vsa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Wave-wide reductions without LDS: DPP within 16-lane rows (xor 1, xor 2,
// half-row mirror, row mirror), then the gfx950 cross-row swaps.
template <typename Op>
__device__ inline float wave_reduce(float x, Op op) {
  auto dpp = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value,
                                                      0xf, 0xf, false));
  };
  x = op(x, dpp(x, std::integral_constant<int, 0xB1>{}));   // quad_perm [1,0,3,2]
  x = op(x, dpp(x, std::integral_constant<int, 0x4E>{}));   // quad_perm [2,3,0,1]
  x = op(x, dpp(x, std::integral_constant<int, 0x141>{}));  // row_half_mirror
  x = op(x, dpp(x, std::integral_constant<int, 0x140>{}));  // row_mirror
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float wave_max(float x) {
  return wave_reduce(x, [](float a, float b) { return fmaxf(a, b); });
}
__device__ inline float wave_sum(float x) {
  return wave_reduce(x, [](float a, float b) { return a + b; });
}

// Order-preserving key of an fp32 score: a > b  <=>  key(a) > key(b); -0 == +0.
__device__ inline uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline void store_out(float* p, float x) { *p = x; }
__device__ inline void store_out(uint16_t* p, float x) { *p = f32_to_bf16_rne(x); }

constexpr int kRows = 16;
// Row tiles up to which the forward splits O_coarse and top-K into separate
// workgroups: the CU count of an MI355X.
constexpr int kSplitTiles = 256;

constexpr int kWaves = 16;  // backward kernels: 1024 threads (<= 128 VGPRs)
// Forward kernel: 1024 threads, one statistics / top-K row per wave.
constexpr int kFwdWaves = 16;

// 16x16 fp32 tile out[r][j] = dot(A row r, B row j) over D, with the D/4
// MFMA steps spread over 4 independent accumulators (short dependency chains).
// brow is always a real row: callers clamp indices past the last cube, and the
// tile entries they produce are never consumed.  Unguarded loads keep the
// compiler from wrapping each one in its own branch.
template <int D>
__device__ __forceinline__ f32x4 dot_tile(const float4 (&af)[D / 16],
                                          const float* __restrict__ brow, int lg) {
  f32x4 acc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f},
                  {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  float4 bf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    bf[kk] = *reinterpret_cast<const float4*>(brow + 16 * kk + 4 * lg);
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[kk].x, bf[kk].x, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[kk].y, bf[kk].y, acc[1], 0, 0, 0);
    acc[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[kk].z, bf[kk].z, acc[2], 0, 0, 0);
    acc[3] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[kk].w, bf[kk].w, acc[3], 0, 0, 0);
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// KPL: keys per lane in the top-K, ceil(C / 64) rounded up to a power of two.
// R: query-cube rows per workgroup, 16, or 8 above 2048 cubes so that the
// R x C score tile fits in LDS (the 16-row MFMA tiles then repeat the 8 rows
// and drop the repeated half of each result; waves R..15 take no top-K row).
template <typename TOut, int D, int KPL, int R>
__global__ __launch_bounds__(64 * kFwdWaves) void coarse_kernel(const float* __restrict__ qm,
                                                               const float* __restrict__ km,
                                                               const float* __restrict__ vm,
                                                               TOut* __restrict__ oc,
                                                               int32_t* __restrict__ idx,
                                                               float* __restrict__ scores, Geo g,
                                                               int ldc) {
  constexpr int kOcWaves = D / 16;                // 16-wide slices of O_coarse
  constexpr int kHalves = kFwdWaves / kOcWaves;   // waves sharing one slice, over key batches
  constexpr int kQS = D + 4;                      // padded row stride of qs (floats)
  extern __shared__ float lds[];
  float* sc = lds;                       // [R][ldc]
  float* rowmax = lds + R * ldc;         // [R]
  float* rowinv = rowmax + R;            // [R]
  float* qs = rowinv + R;                // [R][kQS]: the query rows, loaded once
  float* part = qs + R * kQS;            // [kFwdWaves - kOcWaves][64][4]: O_coarse partial sums

  constexpr float kScale = (D == 64) ? 0.125f : 0.08838834764831845f;  // 1/sqrt(D)
  const int C = g.C;
  const int64_t bh = blockIdx.y;
  const int row0 = blockIdx.x * R;
  // split grid: z = 0 statistics and O_coarse, z = 1 top-K; otherwise both
  const bool both = gridDim.z == 1;
  const bool oc_role = blockIdx.z == 0;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const float* qh = qm + bh * C * D;
  const float* kh = km + bh * C * D;
  const float* vh = vm + bh * C * D;
  const int dt = wave % kOcWaves, half = wave / kOcWaves;

  // Vc operand of this wave's first key batch (O_coarse workgroups), issued
  // now so that its latency overlaps the score phase.  Lane (li, lg) feeds
  // B[k=lg][n=li] = Vc[j][16*dt + li] for j = j0 + 16(u/4) + 4lg + u%4.
  float b[16];
  auto load_batch = [&](int j0) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int j = j0 + 16 * (u >> 2) + 4 * lg + (u & 3);
      b[u] = vh[(int64_t)min(j, C - 1) * D + dt * 16 + li];   // j >= C: weight 0 below
    }
  };
  if (oc_role) load_batch(64 * half);

  // -- 1. scores.  Lane (li, lg) feeds A[m=li][k=lg] and B[k=lg][n=li]; the
  // t-th of four MFMAs per 16-wide slice of D uses d = 16*kk + 4*lg + t for
  // both operands, so their products pair up on the same d.
  // The 16 query rows are read from memory once, coalesced, into LDS: every
  // scoring wave needs all of them, and a per-wave load would fetch them 16
  // times over the workgroup's vector memory path.
  for (int e = threadIdx.x; e < R * D / 4; e += 64 * kFwdWaves) {
    const int r = e / (D / 4), c4 = e % (D / 4);
    const float4 x = (row0 + r < C) ? *reinterpret_cast<const float4*>(qh + (int64_t)(row0 + r) * D + 4 * c4)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(qs + r * kQS + 4 * c4) = x;
  }
  __syncthreads();
  const int ntile = (C + 15) / 16;
  float4 qf[D / 16];
  if (wave < ntile) {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      qf[kk] = *reinterpret_cast<const float4*>(qs + (li % R) * kQS + 16 * kk + 4 * lg);
  }
  for (int ct = wave; ct < ntile; ct += kFwdWaves) {
    const int col = ct * 16 + li;
    const f32x4 acc = dot_tile<D>(qf, kh + (int64_t)min(col, C - 1) * D, lg);
    // acc[r] is the dot product of query row 4*lg + r with key column col
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = 4 * lg + r;
      if (rr >= R) continue;
      const float s = acc[r] * kScale;
      sc[rr * ldc + col] = s;
      if (oc_role && scores != nullptr && row0 + rr < C && col < C)
        scores[(bh * C + row0 + rr) * C + col] = s;
    }
  }
  __syncthreads();

  if (oc_role) {
    // -- 2. softmax statistics, one row per wave
    for (int rr = wave; rr < R; rr += kFwdWaves) {
      const float* srow = sc + rr * ldc;
      float m = -INFINITY;
      for (int j = lane; j < C; j += 64) m = fmaxf(m, srow[j]);
      m = wave_max(m);
      float s = 0.f;
      for (int j = lane; j < C; j += 64) s += __expf(srow[j] - m);
      s = wave_sum(s);
      if (lane == 0) {
        rowmax[rr] = m;
        rowinv[rr] = 1.f / s;
      }
    }
    __syncthreads();

    // -- 3. O_coarse = P Vc: A[m=li][k=lg] = P[row li][j], B[k=lg][n=li] = Vc[j][col].
    // The kHalves waves of a slice take every kHalves-th batch of 64 keys;
    // each batch of 16 Vc loads is issued one batch ahead of its MFMAs, and
    // the 16 MFMAs of a batch alternate between 4 accumulators.
    const float mrow = rowmax[li % R], irow = rowinv[li % R];
    const float* prow = sc + (li % R) * ldc;
    f32x4 acc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f},
                    {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    for (int j0 = 64 * half; j0 < C; j0 += 64 * kHalves) {
      float bc[16], a[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) bc[u] = b[u];
      if (j0 + 64 * kHalves < C) load_batch(j0 + 64 * kHalves);
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int j = j0 + 16 * (u >> 2) + 4 * lg + (u & 3);
        const float e = __expf(prow[min(j, C - 1)] - mrow) * irow;
        a[u] = (j < C) ? e : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u)
        acc[u & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u], bc[u], acc[u & 3], 0, 0, 0);
    }
    const f32x4 tot = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    // the slice's partial sums meet in LDS, added in a fixed order
    if (half > 0) *reinterpret_cast<f32x4*>(part + ((wave - kOcWaves) * 64 + lane) * 4) = tot;
    __syncthreads();
    if (half == 0) {
      f32x4 sum = tot;
#pragma unroll
      for (int h = 1; h < kHalves; ++h)
        sum += *reinterpret_cast<const f32x4*>(part + (((h - 1) * kOcWaves + dt) * 64 + lane) * 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + 4 * lg + r;
        if (4 * lg + r < R && row < C) store_out(oc + (bh * C + row) * D + dt * 16 + li, sum[r]);
      }
    }
    if (!both) return;
  }

  // -- 4. top-K, one row per wave.  Counting a predicate over the row is one
  // 64-bit ballot plus a scalar popcount per 64 keys.
  static_assert(R <= kFwdWaves, "one top-K row per wave");
  const int rr = wave;
  if (rr >= R || row0 + rr >= C) return;
  const int K = g.K;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const float* srow = sc + rr * ldc;
  uint32_t key[KPL];
#pragma unroll
  for (int e = 0; e < KPL; ++e) {
    const int j = e * 64 + lane;
    key[e] = (j < C) ? score_key(srow[j]) : 0u;  // 0 is below every score key
  }
  // largest threshold t with #{key >= t} >= K, i.e. the K-th largest key
  uint32_t thr = 0u;
#pragma unroll 8
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < KPL; ++e) cnt += __popcll(__ballot(key[e] >= cand));
    if (cnt >= K) thr = cand;
  }
  int gt = 0;
#pragma unroll
  for (int e = 0; e < KPL; ++e) gt += __popcll(__ballot(key[e] > thr));
  const int need = K - gt;  // ties at the threshold to keep, lowest index first
  int ties_before = 0, sel_before = 0;
  int32_t* out = idx + (bh * C + row0 + rr) * K;
#pragma unroll
  for (int e = 0; e < KPL; ++e) {
    const int j = e * 64 + lane;
    const bool is_gt = (j < C) && key[e] > thr;
    const bool is_eq = (j < C) && key[e] == thr;
    const uint64_t eqm = __ballot(is_eq);
    const int eq_rank = ties_before + __popcll(eqm & lt_mask);
    const bool take = is_gt || (is_eq && eq_rank < need);
    const uint64_t takem = __ballot(take);
    if (take) out[sel_before + __popcll(takem & lt_mask)] = j;
    ties_before += __popcll(eqm);
    sel_before += __popcll(takem);
  }
}

template <typename TOut, int D, int KPL, int R>
hipError_t launch_kpl(const Geo& g, const float* qm, const float* km, const float* vm, void* oc,
                      int32_t* idx, float* scores, hipStream_t s) {
  const int ntile = (g.C + 15) / 16;
  const int ldc = ntile * 16 + 1;  // odd stride spreads a column over the LDS banks
  const size_t lds = (size_t)(R * ldc + 2 * R + R * (D + 4) +
                              (kFwdWaves - D / 16) * 64 * 4) * sizeof(float);
  auto* kern = coarse_kernel<TOut, D, KPL, R>;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  // two workgroups per row tile while one per tile leaves CUs idle
  const int rtiles = (g.C + R - 1) / R;
  const int roles = int64_t(rtiles) * g.B * g.H <= kSplitTiles ? 2 : 1;
  return launch_kernel(kern, dim3(rtiles, g.B * g.H, roles), dim3(64 * kFwdWaves), lds, s, qm, km,
                       vm, static_cast<TOut*>(oc), idx, scores, g, ldc);
}

template <typename TOut, int D>
hipError_t launch_typed(const Geo& g, const float* qm, const float* km, const float* vm,
                        void* oc, int32_t* idx, float* scores, hipStream_t s) {
  static_assert(kMaxCubes <= 64 * 64, "top-K holds at most 64 keys per lane");
  const int per_lane = (g.C + 63) / 64;
  if (per_lane <= 1) return launch_kpl<TOut, D, 1, 16>(g, qm, km, vm, oc, idx, scores, s);
  if (per_lane <= 2) return launch_kpl<TOut, D, 2, 16>(g, qm, km, vm, oc, idx, scores, s);
  if (per_lane <= 4) return launch_kpl<TOut, D, 4, 16>(g, qm, km, vm, oc, idx, scores, s);
  if (per_lane <= 8) return launch_kpl<TOut, D, 8, 16>(g, qm, km, vm, oc, idx, scores, s);
  if (per_lane <= 16) return launch_kpl<TOut, D, 16, 16>(g, qm, km, vm, oc, idx, scores, s);
  if (per_lane <= 32) return launch_kpl<TOut, D, 32, 16>(g, qm, km, vm, oc, idx, scores, s);
  return launch_kpl<TOut, D, 64, 8>(g, qm, km, vm, oc, idx, scores, s);
}

// ---------------------------------------------------------------------------
// Backward of the coarse stage.  With Pc = softmax(Sc), Sc = Qc Kc^T / sqrt(D)
// and dOc the per-cube sums of dO_coarse:
//   dPc = dOc Vc^T,  dSc = Pc * (dPc - rowsum(Pc * dPc)),
//   dQc = dSc Kc / sqrt(D),  dKc = dSc^T Qc / sqrt(D),  dVc = Pc^T dOc.
// Row pass (16 query cubes per workgroup): dQc and the per-row statistics.
// Column pass (16 key cubes per workgroup): dKc and dVc, recomputing Pc and
// dSc column-wise from those statistics.  Both are deterministic.

// out1[r][j] = scale1 * dot(A1[r], B1[j]) and out2[r][j] = dot(A2[r], B2[j])
// for the 16 rows r starting at a0 and every j of the 16-aligned column
// range, into LDS with row stride ldc.  The 2 x 16 A rows are read from
// memory once, coalesced, into `stage` (which may overlap out1/out2: every
// wave takes its operands into registers before any output is written) —
// a per-wave load would fetch them once per wave.  Rows and columns past
// the last cube repeat the last one (finite values no later step consumes).
// R rows per workgroup (16, or 8 for large C so that two R x C score tiles
// fit in LDS): with R = 8 the 16-row MFMA tiles repeat the 8 rows and the
// repeated half of each result is dropped.
template <int D, int R>
__device__ __forceinline__ void rows_dot2(const float* __restrict__ A1,
                                          const float* __restrict__ A2, int a0,
                                          const float* __restrict__ B1,
                                          const float* __restrict__ B2, int C, float scale1,
                                          float* out1, float* out2, int ldc, float* stage,
                                          int wave, int lane) {
  constexpr int kAS = D + 4;   // padded row stride of the staged rows (floats)
  const int li = lane & 15, lg = lane >> 4;
  for (int e = threadIdx.x; e < 2 * R * D / 4; e += 64 * kWaves) {
    const int t = e / (R * D / 4), rem = e % (R * D / 4);
    const int r = rem / (D / 4), c4 = rem % (D / 4);
    const float* A = t ? A2 : A1;
    const float4 x = *reinterpret_cast<const float4*>(A + (int64_t)min(a0 + r, C - 1) * D + 4 * c4);
    *reinterpret_cast<float4*>(stage + (t * R + r) * kAS + 4 * c4) = x;
  }
  __syncthreads();
  // task = (product, column tile): even waves take product 1, odd waves 2
  const int prod = wave & 1;
  float4 af[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    af[kk] = *reinterpret_cast<const float4*>(stage + (prod * R + li % R) * kAS + 16 * kk + 4 * lg);
  __syncthreads();
  const int ntile = (C + 15) / 16;
  const float* const B = prod ? B2 : B1;
  float* const out = prod ? out2 : out1;
  const float scale = prod ? 1.f : scale1;
  for (int ct = wave >> 1; ct < ntile; ct += kWaves / 2) {
    const int col = ct * 16 + li;
    const int64_t cc = min(col, C - 1);
    const f32x4 acc = dot_tile<D>(af, B + cc * D, lg);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      if (4 * lg + rr < R) out[(4 * lg + rr) * ldc + col] = acc[rr] * scale;
  }
}

// y[r][:] = scale * sum_j T[r][j] Y[j][:] for the R LDS rows of T, stored to
// out rows o0 + r (< C) of an fp32 [C][D] matrix.
template <int D, int R>
__device__ __forceinline__ void lds_times(const float* T, int ldc, const float* __restrict__ Y,
                                          int C, float scale, float* __restrict__ out, int o0,
                                          int wave, int lane, int nwaves) {
  const int li = lane & 15, lg = lane >> 4;
  const float* trow = T + (li % R) * ldc;
  for (int dt = wave; dt < D / 16; dt += nwaves) {
    f32x4 acc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f},
                    {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    // each batch of 16 Y loads is issued one batch ahead of its MFMAs
    float b[16];
    auto load_batch = [&](int j0) {
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int j = j0 + 16 * (u >> 2) + 4 * lg + (u & 3);
        b[u] = Y[(int64_t)min(j, C - 1) * D + dt * 16 + li];   // j >= C: weight 0 below
      }
    };
    load_batch(0);
    for (int j0 = 0; j0 < C; j0 += 64) {
      float a[16], bc[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) bc[u] = b[u];
      if (j0 + 64 < C) load_batch(j0 + 64);
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int j = j0 + 16 * (u >> 2) + 4 * lg + (u & 3);
        const float t = trow[min(j, C - 1)];
        a[u] = (j < C) ? t : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u)
        acc[u & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u], bc[u], acc[u & 3], 0, 0, 0);
    }
    const f32x4 tot = (acc[0] + acc[1]) + (acc[2] + acc[3]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = o0 + 4 * lg + r;
      if (4 * lg + r < R && row < C) out[(int64_t)row * D + dt * 16 + li] = tot[r] * scale;
    }
  }
}

// With lists.idx set, the last workgroup column builds the transposed block
// lists of its head instead (spare workgroups of this small grid).
struct ListArgs {
  const int32_t* idx; int32_t* offsets; int32_t* list; int32_t* order;
};
static_assert(64 * kWaves == kBitmapThreads, "block-list workgroups have the row kernel's size");

template <int D, int R>
__global__ __launch_bounds__(64 * kWaves) void coarse_bwd_rows_kernel(
    const float* __restrict__ qm, const float* __restrict__ km, const float* __restrict__ vm,
    const float* __restrict__ docs, float* __restrict__ stats, float* __restrict__ dqc, Geo g,
    int ldc, ListArgs lists) {
  extern __shared__ float lds[];
  if (lists.idx != nullptr && blockIdx.x == gridDim.x - 1) {
    idx_transpose_bitmap(lists.idx, lists.offsets, lists.list, lists.order, g, blockIdx.y,
                         reinterpret_cast<uint32_t*>(lds));
    return;
  }
  float* s1 = lds;                 // scores, then probabilities
  float* s2 = lds + R * ldc;       // dPc, then dSc
  constexpr float kScale = (D == 64) ? 0.125f : 0.08838834764831845f;
  const int C = g.C;
  const int64_t bh = blockIdx.y;
  const int row0 = blockIdx.x * R;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t hoff = bh * C * D;
  rows_dot2<D, R>(qm + hoff, docs + hoff, row0, km + hoff, vm + hoff, C, kScale, s1, s2, ldc, lds,
                  wave, lane);
  __syncthreads();
  for (int rr = wave; rr < R; rr += kWaves) {
    float* p = s1 + rr * ldc;
    float* dp = s2 + rr * ldc;
    float m = -INFINITY;
    for (int j = lane; j < C; j += 64) m = fmaxf(m, p[j]);
    m = wave_max(m);
    float l = 0.f;
    for (int j = lane; j < C; j += 64) l += __expf(p[j] - m);
    l = wave_sum(l);
    const float inv = 1.f / l;
    float r = 0.f;
    for (int j = lane; j < C; j += 64) {
      const float pj = __expf(p[j] - m) * inv;
      p[j] = pj;
      r += pj * dp[j];
    }
    r = wave_sum(r);
    for (int j = lane; j < C; j += 64) dp[j] = p[j] * (dp[j] - r);
    if (lane == 0 && row0 + rr < C) {
      const int64_t at = bh * C + row0 + rr;
      stats[at] = m;
      stats[(int64_t)g.B * g.H * C + at] = l;
      stats[2 * (int64_t)g.B * g.H * C + at] = r;
    }
  }
  __syncthreads();
  lds_times<D, R>(s2, ldc, km + hoff, C, kScale, dqc + hoff, row0, wave, lane, kWaves);
}

template <int D, int R>
__global__ __launch_bounds__(64 * kWaves) void coarse_bwd_cols_kernel(
    const float* __restrict__ qm, const float* __restrict__ km, const float* __restrict__ vm,
    const float* __restrict__ docs, const float* __restrict__ stats, float* __restrict__ dkc,
    float* __restrict__ dvc, Geo g, int ldc) {
  extern __shared__ float lds[];
  float* t1 = lds;                 // Sc^T rows (R key cubes x C query cubes), then Pc^T
  float* t2 = lds + R * ldc;       // dPc^T, then dSc^T
  constexpr float kScale = (D == 64) ? 0.125f : 0.08838834764831845f;
  const int C = g.C;
  const int64_t bh = blockIdx.y;
  const int col0 = blockIdx.x * R;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t hoff = bh * C * D;
  rows_dot2<D, R>(km + hoff, vm + hoff, col0, qm + hoff, docs + hoff, C, kScale, t1, t2, ldc, lds,
                  wave, lane);
  __syncthreads();
  const int64_t plane = (int64_t)g.B * g.H * C;
  const float* sm = stats + bh * C;
  const float* sl = sm + plane;
  const float* sr = sm + 2 * plane;
  for (int e = threadIdx.x; e < R * C; e += 64 * kWaves) {
    const int jj = e / C, i = e % C;
    const float p = __expf(t1[jj * ldc + i] - sm[i]) / sl[i];
    t1[jj * ldc + i] = p;
    t2[jj * ldc + i] = p * (t2[jj * ldc + i] - sr[i]);
  }
  __syncthreads();
  // dKc on one half of the waves, dVc on the other
  constexpr int kHalf = kWaves / 2;
  if (wave < kHalf) lds_times<D, R>(t2, ldc, qm + hoff, C, kScale, dkc + hoff, col0, wave, lane, kHalf);
  else lds_times<D, R>(t1, ldc, docs + hoff, C, 1.f, dvc + hoff, col0, wave - kHalf, lane, kHalf);
}

template <int D, int R>
hipError_t launch_coarse_bwd_typed(const Geo& g, const float* qm, const float* km,
                                   const float* vm, const float* docs, float* stats,
                                   float* dqc, float* dkc, float* dvc, const ListArgs& lists,
                                   hipStream_t s) {
  const int ntile = (g.C + R - 1) / R;          // row (column) tiles of R cubes
  const int ldc = (g.C + 15) / 16 * 16 + 1;     // scores are computed in 16-column tiles
  // two R x C score tiles, or the 2 x R staged operand rows if larger
  size_t lds = (size_t)std::max(2 * R * ldc, 2 * R * (D + 4)) * sizeof(float);
  if (lists.idx != nullptr) lds = std::max(lds, bitmap_words(g.C) * sizeof(uint32_t));
  auto* rows = coarse_bwd_rows_kernel<D, R>;
  auto* cols = coarse_bwd_cols_kernel<D, R>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(rows),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(cols),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const dim3 grid(ntile, g.B * g.H), block(64 * kWaves);
  const dim3 rows_grid(ntile + (lists.idx != nullptr ? 1 : 0), g.B * g.H);
  hipError_t e = launch_kernel(rows, rows_grid, block, lds, s, qm, km, vm, docs, stats, dqc, g,
                               ldc, lists);
  if (e != hipSuccess) return e;
  return launch_kernel(cols, grid, block, lds, s, qm, km, vm, docs,
                       static_cast<const float*>(stats), dkc, dvc, g, ldc);
}

}  // namespace

hipError_t launch_coarse(const Geo& g, int dtype, const float* qm, const float* km,
                         const float* vm, void* oc, int32_t* idx, float* scores,
                         hipStream_t s) {
  if (dtype == 1)
    return g.D == 128 ? launch_typed<uint16_t, 128>(g, qm, km, vm, oc, idx, scores, s)
                      : launch_typed<uint16_t, 64>(g, qm, km, vm, oc, idx, scores, s);
  return g.D == 128 ? launch_typed<float, 128>(g, qm, km, vm, oc, idx, scores, s)
                    : launch_typed<float, 64>(g, qm, km, vm, oc, idx, scores, s);
}

}  // namespace vsa

namespace vsa {

hipError_t launch_coarse_bwd(const Geo& g, const float* qm, const float* km, const float* vm,
                             const float* docs, float* stats, float* dqc, float* dkc,
                             float* dvc, const int32_t* idx, int32_t* offsets, int32_t* list,
                             int32_t* order, hipStream_t s) {
  const ListArgs lists = {g.C <= kBitmapCubes ? idx : nullptr, offsets, list, order};
  // 16 cubes per workgroup while two 16 x C fp32 tiles fit the LDS, else 8,
  // else 4; small grids take 8 (more workgroups: at 112 cubes and 12 heads
  // the backward is 1.5 us faster than with 16, the forward's coarse kernel
  // is not)
  if (g.C > kCoarseBwd8Cubes)
    return g.D == 128
               ? launch_coarse_bwd_typed<128, 4>(g, qm, km, vm, docs, stats, dqc, dkc, dvc, lists, s)
               : launch_coarse_bwd_typed<64, 4>(g, qm, km, vm, docs, stats, dqc, dkc, dvc, lists, s);
  if (g.C > kCoarseBwdSmallCubes && g.C <= kCoarseBwd16Cubes)
    return g.D == 128
               ? launch_coarse_bwd_typed<128, 16>(g, qm, km, vm, docs, stats, dqc, dkc, dvc, lists, s)
               : launch_coarse_bwd_typed<64, 16>(g, qm, km, vm, docs, stats, dqc, dkc, dvc, lists, s);
  return g.D == 128
             ? launch_coarse_bwd_typed<128, 8>(g, qm, km, vm, docs, stats, dqc, dkc, dvc, lists, s)
             : launch_coarse_bwd_typed<64, 8>(g, qm, km, vm, docs, stats, dqc, dkc, dvc, lists, s);
}

}  // namespace vsa
