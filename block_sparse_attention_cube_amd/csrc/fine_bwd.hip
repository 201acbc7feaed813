// Backward of VSA (the trainable path): preparation pass, transposed block
// lists, and the two fine-stage gradient kernels.
//
// With S = Q K^T / sqrt(d) over the selected blocks, P = exp(S - lse) and
// D = rowsum(dO * O):
//   dV_j = sum_i P_ij^T dO_i,  dP = dO V^T,  dS = P * (dP - D),
//   dQ_i = sum_j dS_ij K_j / sqrt(d),  dK_j = sum_i dS_ij^T Q_i / sqrt(d).
// dQ is produced per query cube (loop over its K selected key cubes), dK/dV
// per key cube (loop over the query cubes that selected it, from a counting
// sort of the index list).  Neither kernel uses atomics, so results are
// bit-reproducible.  Each kernel adds the coarse-stage gradient of its cube
// (divided by the cube's valid-token count) and writes raster rows.
//
// Both kernels follow the forward's MFMA layouts (v_mfma_f32_16x16x32_bf16,
// scores kept in the accumulator layout of the transposed product so that
// probabilities feed the next MFMA straight from registers); operands whose
// contraction index is the token index are staged transposed in LDS.
#include "vsa_internal.h"
#include "vsa_bwd.h"

namespace vsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

template <int D>
constexpr float inv_sqrt_d() { return D == 64 ? 0.125f : 0.08838834764831845f; }

__device__ inline bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}
__device__ inline uint32_t lo_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ inline uint32_t hi_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Column of token kappa in a transposed row: tokens 32s + 16h + 4g + r go
// to 32s + 8g + 4h + r, so the 8 tokens one lane feeds to an MFMA k-step
// ({32s + 4g + r} and {32s + 16 + 4g + r}) end up in one 16-byte run.
__device__ constexpr int tr_col(int kappa) {
  return (kappa & ~31) | (((kappa >> 2) & 3) << 3) | (((kappa >> 4) & 1) << 2) | (kappa & 3);
}
constexpr int kTrStride = 72;   // transposed rows: 64 tokens + 8 pad (144 bytes)

// One 64-token block staged twice in LDS: row-major [64][D] (16-byte chunks
// XOR-swizzled by row) and transposed [D][72] in tr_col order.  A thread
// moves 4 tokens x 8 dims: token 4*tg + u, dims 8*dc .. 8*dc + 7.
template <int D>
struct BlockStage {
  static constexpr int kRowElems = 64 * D;
  static constexpr int kTrElems = D * kTrStride;
  static constexpr int kThreads = 2 * D;   // 16 token groups x D/8 dim chunks
  u32x4 r[4];
  int tid, tg, dc;
  __device__ __forceinline__ void init(int t) { tid = t; tg = t % 16; dc = t / 16; }
  __device__ __forceinline__ void load(const uint16_t* __restrict__ src) {
    if (tid < kThreads) {
      const uint16_t* b = src + (4 * tg) * D + 8 * dc;
#pragma unroll
      for (int u = 0; u < 4; ++u) r[u] = *reinterpret_cast<const u32x4*>(b + u * D);
    }
  }
  __device__ __forceinline__ void store_rows(uint16_t* rows) const {
    constexpr int kKC = D / 8;
    if (tid < kThreads) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int row = 4 * tg + u;
        *reinterpret_cast<u32x4*>(rows + row * D + ((dc ^ (row & (kKC - 1))) * 8)) = r[u];
      }
    }
  }
  __device__ __forceinline__ void store_tr(uint16_t* tr) const {
    if (tid < kThreads) {
      const int col = tr_col(4 * tg);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int d0 = 8 * dc + 2 * h;
        const u32x2 lo = {lo_lo(r[0][h], r[1][h]), lo_lo(r[2][h], r[3][h])};
        const u32x2 hi = {hi_hi(r[0][h], r[1][h]), hi_hi(r[2][h], r[3][h])};
        *reinterpret_cast<u32x2*>(tr + d0 * kTrStride + col) = lo;
        *reinterpret_cast<u32x2*>(tr + (d0 + 1) * kTrStride + col) = hi;
      }
    }
  }
};

// Row-major operand read: 8 consecutive dims of token `row` starting at chunk c.
template <int D>
__device__ __forceinline__ u32x4 read_row(const uint16_t* rows, int row, int c) {
  constexpr int kKC = D / 8;
  return *reinterpret_cast<const u32x4*>(rows + row * D + ((c ^ (row & (kKC - 1))) * 8));
}

// Writes a [64][D] fp32 tile held in MFMA accumulators to raster rows of a
// cube through LDS, adding an fp32 per-cube row `extra` (scaled by inv_n).
// get(row, d) is evaluated by the owning lane; here the caller has already
// written bf16 rows into `stage` ([64][D+8]).
template <int D>
__device__ __forceinline__ void write_cube_rows(const uint16_t* stage, uint16_t* __restrict__ out,
                                                const Geo& g, int64_t bh, int c, int tid) {
  constexpr int kKC = D / 8, kOS = D + 8, kOutReg = 64 * kKC / 256;
  const CubeExt e = cube_extent(g, c);
#pragma unroll
  for (int u = 0; u < kOutReg; ++u) {
    const int ch = tid + 256 * u, row = ch / kKC, cc = ch % kKC;
    const int64_t tok = slot_token(g, e, row);
    if (tok >= 0)
      *reinterpret_cast<u32x4*>(out + (bh * g.N + tok) * D + 8 * cc) =
          *reinterpret_cast<const u32x4*>(stage + row * kOS + 8 * cc);
  }
}

// ---------------------------------------------------------------------------
// Preparation: raster q, k, v, dO -> cube order; D = rowsum(dO * O) per slot;
// per-cube means of q, k, v and the per-cube sum of dO_coarse.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdPrepArgs a, Geo g) {
  constexpr int kCpr = D / 8;                  // 16-byte chunks per row
  constexpr int kRowsPerPass = 256 / kCpr;
  constexpr int kPasses = kSlots / kRowsPerPass;
  const int c = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const CubeExt e = cube_extent(g, c);
  const int tid = threadIdx.x, chunk = tid % kCpr, row0 = tid / kCpr;
  const uint16_t* src[4] = {a.q, a.k, a.v, a.dof};
  uint16_t* dst[4] = {a.qc, a.kc, a.vc, a.dofc};
  float acc[4][8];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[t][i] = 0.f;

#pragma unroll
  for (int u = 0; u < kPasses; ++u) {
    const int s = row0 + u * kRowsPerPass;
    const int64_t r = slot_token(g, e, s);
    const int64_t crow = bh * g.Np + static_cast<int64_t>(c) * kSlots + s;
    const int64_t rrow = bh * g.N + r;
    u32x4 val[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      val[t] = (r >= 0) ? *reinterpret_cast<const u32x4*>(src[t] + rrow * D + chunk * 8)
                        : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(dst[t] + crow * D + chunk * 8) = val[t];
    }
    const u32x4 ov = (r >= 0) ? *reinterpret_cast<const u32x4*>(a.o + rrow * D + chunk * 8)
                              : u32x4{0u, 0u, 0u, 0u};
    const u32x4 cv = (r >= 0 && a.doc != nullptr)
                         ? *reinterpret_cast<const u32x4*>(a.doc + rrow * D + chunk * 8)
                         : u32x4{0u, 0u, 0u, 0u};
    float dot = 0.f;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      dot = fmaf(bf16_lo(val[3][h]), bf16_lo(ov[h]), dot);
      dot = fmaf(bf16_hi(val[3][h]), bf16_hi(ov[h]), dot);
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        acc[t][2 * h] += bf16_lo(val[t][h]);
        acc[t][2 * h + 1] += bf16_hi(val[t][h]);
      }
      acc[3][2 * h] += bf16_lo(cv[h]);
      acc[3][2 * h + 1] += bf16_hi(cv[h]);
    }
#pragma unroll
    for (int o = kCpr / 2; o >= 1; o >>= 1) dot += __shfl_xor(dot, o);
    if (chunk == 0) a.delta[crow] = dot;
  }

  __shared__ float red[4][kRowsPerPass][D];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 8; ++i) red[t][row0][chunk * 8 + i] = acc[t][i];
  __syncthreads();
  if (tid < D) {
    const float inv_n = 1.f / static_cast<float>(e.nt * e.nh * e.nw);
    float sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rr = 0; rr < kRowsPerPass; ++rr)
#pragma unroll
      for (int t = 0; t < 4; ++t) sum[t] += red[t][rr][tid];
    const int64_t m = (bh * g.C + c) * D + tid;
    a.qm[m] = sum[0] * inv_n;
    a.km[m] = sum[1] * inv_n;
    a.vm[m] = sum[2] * inv_n;
    a.docs[m] = sum[3];
  }
}

// ---------------------------------------------------------------------------
// Transposed block lists: for each key cube j of head (b, h), the query cubes
// whose selection contains j, in ascending order.  One workgroup per head:
// count, exclusive scan, then rows are placed R at a time (R <= 32): every
// entry sets its row's bit in a per-key mask (atomicOr, order-free), and its
// position is the key's cursor plus the number of earlier rows of the step
// that hold the same key -- deterministic, no ordering by atomics.
__global__ __launch_bounds__(256) void idx_transpose_kernel(const int32_t* __restrict__ idx,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ list, Geo g) {
  extern __shared__ int32_t shared[];
  int32_t* cursor = shared;                                   // [C] counts, then cursors
  uint32_t* mask = reinterpret_cast<uint32_t*>(shared + g.C);  // [C] rows of this step
  __shared__ int32_t part[256];
  const int64_t bh = blockIdx.x;
  const int C = g.C, K = g.K, tid = threadIdx.x;
  const int32_t* rows = idx + bh * C * K;
  for (int j = tid; j < C; j += 256) {
    cursor[j] = 0;
    mask[j] = 0u;
  }
  __syncthreads();
  for (int e = tid; e < C * K; e += 256) atomicAdd(&cursor[rows[e]], 1);
  __syncthreads();
  // exclusive scan of the C counts: per-thread chunk sums, serial scan of 256 partials
  const int per = (C + 255) / 256;
  const int lo = min(C, tid * per), hi = min(C, lo + per);
  int sum = 0;
  for (int j = lo; j < hi; ++j) sum += cursor[j];
  part[tid] = sum;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int t = 0; t < 256; ++t) {
      const int x = part[t];
      part[t] = run;
      run += x;
    }
  }
  __syncthreads();
  int run = part[tid];
  int32_t* off = offsets + bh * (C + 1);
  for (int j = lo; j < hi; ++j) {
    const int x = cursor[j];
    cursor[j] = run;
    off[j] = run;
    run += x;
  }
  if (tid == 0) off[C] = C * K;
  __syncthreads();
  int32_t* out = list + bh * C * K;
  const int R = max(1, min(32, 256 / K));
  for (int i0 = 0; i0 < C; i0 += R) {
    const int n = min(R, C - i0) * K;
    for (int e = tid; e < n; e += 256) atomicOr(&mask[rows[i0 * K + e]], 1u << (e / K));
    __syncthreads();
    for (int e = tid; e < n; e += 256) {
      const int r = e / K, j = rows[i0 * K + e];
      out[cursor[j] + __popc(mask[j] & ((1u << r) - 1u))] = i0 + r;
    }
    __syncthreads();
    for (int j = tid; j < C; j += 256) {
      cursor[j] += __popc(mask[j]);
      mask[j] = 0u;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per query cube, 4 waves x 16 query slots (as the forward).
template <int D>
__global__ __launch_bounds__(256, 2) void fine_bwd_dq_kernel(BwdFineArgs a, Geo g) {
  constexpr int kKS = D / 32, kDT = D / 16, kOS = D + 8;
  using Stage = BlockStage<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * Stage::kRowElems + Stage::kTrElems];
  uint16_t* const k_rows = smem;
  uint16_t* const v_rows = smem + Stage::kRowElems;
  uint16_t* const k_tr = smem + 2 * Stage::kRowElems;

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bh = tile / g.C;
  const int qc = tile % g.C;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int K = g.K;
  const int32_t* __restrict__ sel = a.idx + static_cast<int64_t>(tile) * K;
  const float c2 = inv_sqrt_d<D>() * kLog2e;
  const int64_t qrow = bh * g.Np + static_cast<int64_t>(qc) * 64 + wave * 16 + li;

  u32x4 qf[kKS], df[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    qf[ks] = *reinterpret_cast<const u32x4*>(a.qc + qrow * D + 32 * ks + 8 * lg);
    df[ks] = *reinterpret_cast<const u32x4*>(a.dofc + qrow * D + 32 * ks + 8 * lg);
  }
  const float lse2 = a.lse[qrow] * kLog2e;
  const float delta = a.delta[qrow];

  Stage ks_, vs_;
  ks_.init(tid);
  vs_.init(tid);
  f32x4 dacc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) dacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  int64_t base = (bh * g.Np + static_cast<int64_t>(sel[0]) * 64) * D;
  ks_.load(a.kc + base);
  vs_.load(a.vc + base);
  for (int n = 0; n < K; ++n) {
    const int j = sel[n];
    ks_.store_rows(k_rows);
    ks_.store_tr(k_tr);
    vs_.store_rows(v_rows);
    __syncthreads();
    if (n + 1 < K) {
      base = (bh * g.Np + static_cast<int64_t>(sel[n + 1]) * 64) * D;
      ks_.load(a.kc + base);
      vs_.load(a.vc + base);
    }
    // S^T and dP^T: lane holds (q = li, key = 16kb + 4lg + r)
    f32x4 sacc[4], pacc[4];
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int row = 16 * kb + li;
        const u32x4 kf = read_row<D>(k_rows, row, 4 * ks + lg);
        const u32x4 vf = read_row<D>(v_rows, row, 4 * ks + lg);
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(kf), as_bf16x8(qf[ks]), ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[kb], 0, 0, 0);
        pacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(vf), as_bf16x8(df[ks]), ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : pacc[kb], 0, 0, 0);
      }
    }
    const CubeExt e = cube_extent(g, j);
    const bool edge = e.nt < 4 || e.nh < 4 || e.nw < 4;
    u32x4 dsf[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float ds[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kb = 2 * s + (i >> 2), r = i & 3;
        float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], c2, -lse2));
        if (edge && (kb >= e.nt || lg >= e.nh || r >= e.nw)) p = 0.f;
        ds[i] = p * (pacc[kb][r] - delta);
      }
      dsf[s] = u32x4{pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]),
                     pack_bf16x2(ds[4], ds[5]), pack_bf16x2(ds[6], ds[7])};
    }
    // dQ^T[d][q] += K^T[d][keys] dS^T[keys][q]
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
        const u32x4 kt =
            *reinterpret_cast<const u32x4*>(k_tr + (16 * dt + li) * kTrStride + 32 * s + 8 * lg);
        dacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kt), as_bf16x8(dsf[s]),
                                                           dacc[dt], 0, 0, 0);
      }
    __syncthreads();
  }

  // epilogue: dq[q][d] = scale * acc + dQc[qc][d] / n_qc
  uint16_t* const stage = smem;
  const CubeExt eq = cube_extent(g, qc);
  const float inv_n = 1.f / static_cast<float>(eq.nt * eq.nh * eq.nw);
  const float* cq = a.dqc == nullptr ? nullptr : a.dqc + (bh * g.C + qc) * D;
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) {
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d = 16 * dt + 4 * lg + r;
      x[r] = dacc[dt][r] * inv_sqrt_d<D>() + (cq ? cq[d] * inv_n : 0.f);
    }
    const u32x2 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    *reinterpret_cast<u32x2*>(stage + (wave * 16 + li) * kOS + 16 * dt + 4 * lg) = w;
  }
  __syncthreads();
  write_cube_rows<D>(stage, a.dq, g, bh, qc, tid);
}

// ---------------------------------------------------------------------------
// dK/dV: one workgroup per key cube, wave w owns keys 16w..16w+15 and loops
// over the query cubes that selected this key cube.
template <int D>
__global__ __launch_bounds__(256, 2) void fine_bwd_dkdv_kernel(BwdFineArgs a, Geo g) {
  constexpr int kKS = D / 32, kDT = D / 16, kOS = D + 8;
  using Stage = BlockStage<D>;
  __shared__ __attribute__((aligned(16)))
      uint16_t smem[2 * Stage::kRowElems + 2 * Stage::kTrElems];
  __shared__ __attribute__((aligned(16))) float stat[2][64];   // lse*log2e, D per query slot
  uint16_t* const q_rows = smem;
  uint16_t* const o_rows = smem + Stage::kRowElems;
  uint16_t* const q_tr = smem + 2 * Stage::kRowElems;
  uint16_t* const o_tr = q_tr + Stage::kTrElems;

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bh = tile / g.C;
  const int kc = tile % g.C;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const float c2 = inv_sqrt_d<D>() * kLog2e;
  const int64_t krow = bh * g.Np + static_cast<int64_t>(kc) * 64 + wave * 16 + li;

  // B operands of S = Q K^T and dP = dO V^T: lane holds (key = 16w + li, dims 32ks + 8lg ..)
  u32x4 kf[kKS], vf[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    kf[ks] = *reinterpret_cast<const u32x4*>(a.kc + krow * D + 32 * ks + 8 * lg);
    vf[ks] = *reinterpret_cast<const u32x4*>(a.vc + krow * D + 32 * ks + 8 * lg);
  }
  f32x4 dkacc[kDT], dvacc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) {
    dkacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dvacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int32_t* off = a.offsets + bh * (g.C + 1);
  const int beg = off[kc], end = off[kc + 1];
  const int32_t* lst = a.list + bh * g.C * g.K;
  Stage qs_, os_;
  qs_.init(tid);
  os_.init(tid);
  float st_lse = 0.f, st_d = 0.f;
  auto fetch = [&](int qcube) {
    const int64_t base = bh * g.Np + static_cast<int64_t>(qcube) * 64;
    qs_.load(a.qc + base * D);
    os_.load(a.dofc + base * D);
    if (tid < 64) {
      st_lse = a.lse[base + tid] * kLog2e;
      st_d = a.delta[base + tid];
    }
  };
  if (beg < end) fetch(lst[beg]);
  for (int n = beg; n < end; ++n) {
    const int qcube = lst[n];
    __syncthreads();   // previous iteration's readers are done
    qs_.store_rows(q_rows);
    qs_.store_tr(q_tr);
    os_.store_rows(o_rows);
    os_.store_tr(o_tr);
    if (tid < 64) {
      stat[0][tid] = st_lse;
      stat[1][tid] = st_d;
    }
    __syncthreads();
    if (n + 1 < end) fetch(lst[n + 1]);

    // S and dP: lane holds (q = 16qb + 4lg + r, key = 16w + li)
    f32x4 sacc[4], pacc[4];
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const int row = 16 * qb + li;
        const u32x4 qa = read_row<D>(q_rows, row, 4 * ks + lg);
        const u32x4 oa = read_row<D>(o_rows, row, 4 * ks + lg);
        sacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(qa), as_bf16x8(kf[ks]), ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[qb], 0, 0, 0);
        pacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(oa), as_bf16x8(vf[ks]), ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : pacc[qb], 0, 0, 0);
      }
    }
    const CubeExt e = cube_extent(g, qcube);
    u32x4 pf[2], dsf[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float p[8], ds[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int qb = 2 * s + (i >> 2), r = i & 3;
        const int q = 16 * qb + 4 * lg + r;
        const bool valid = qb < e.nt && lg < e.nh && r < e.nw;   // pad query slots add nothing
        p[i] = valid ? __builtin_amdgcn_exp2f(fmaf(sacc[qb][r], c2, -stat[0][q])) : 0.f;
        ds[i] = p[i] * (pacc[qb][r] - stat[1][q]);
      }
      pf[s] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                    pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
      dsf[s] = u32x4{pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]),
                     pack_bf16x2(ds[4], ds[5]), pack_bf16x2(ds[6], ds[7])};
    }
    // dV[key][d] += P^T[key][q] dO[q][d];  dK[key][d] += dS^T[key][q] Q[q][d]
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
        const int col = (16 * dt + li) * kTrStride + 32 * s + 8 * lg;
        const u32x4 ot = *reinterpret_cast<const u32x4*>(o_tr + col);
        const u32x4 qt = *reinterpret_cast<const u32x4*>(q_tr + col);
        dvacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pf[s]), as_bf16x8(ot),
                                                            dvacc[dt], 0, 0, 0);
        dkacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(dsf[s]), as_bf16x8(qt),
                                                            dkacc[dt], 0, 0, 0);
      }
  }
  __syncthreads();

  // epilogue: lane holds (key = 16w + 4lg + r, d = 16dt + li)
  const CubeExt ek = cube_extent(g, kc);
  const float inv_n = 1.f / static_cast<float>(ek.nt * ek.nh * ek.nw);
  const float* ck = a.dkc == nullptr ? nullptr : a.dkc + (bh * g.C + kc) * D;
  const float* cv = a.dvc == nullptr ? nullptr : a.dvc + (bh * g.C + kc) * D;
  uint16_t* const stage_k = smem;
  uint16_t* const stage_v = smem + 64 * kOS;
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) {
    const int d = 16 * dt + li;
    const float addk = ck ? ck[d] * inv_n : 0.f;
    const float addv = cv ? cv[d] * inv_n : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = wave * 16 + 4 * lg + r;
      const float xk = dkacc[dt][r] * inv_sqrt_d<D>() + addk;
      const float xv = dvacc[dt][r] + addv;
      stage_k[key * kOS + d] = f32_to_bf16_rne(xk);
      stage_v[key * kOS + d] = f32_to_bf16_rne(xv);
    }
  }
  __syncthreads();
  write_cube_rows<D>(stage_k, a.dk, g, bh, kc, tid);
  write_cube_rows<D>(stage_v, a.dv, g, bh, kc, tid);
}

}  // namespace

hipError_t launch_bwd_prep(const Geo& g, const BwdPrepArgs& a, hipStream_t s) {
  const dim3 grid(g.C, g.B * g.H), block(256);
  return g.D == 128 ? launch_kernel(bwd_prep_kernel<128>, grid, block, 0, s, a, g)
                    : launch_kernel(bwd_prep_kernel<64>, grid, block, 0, s, a, g);
}

hipError_t launch_idx_transpose(const Geo& g, const int32_t* idx, int32_t* offsets,
                                int32_t* list, hipStream_t s) {
  return launch_kernel(idx_transpose_kernel, dim3(g.B * g.H), dim3(256),
                       2 * static_cast<size_t>(g.C) * sizeof(int32_t), s, idx, offsets, list, g);
}

hipError_t launch_bwd_fine(const Geo& g, const BwdFineArgs& a, hipStream_t s) {
  const dim3 grid(g.B * g.H * g.C), block(256);
  hipError_t e = g.D == 128 ? launch_kernel(fine_bwd_dq_kernel<128>, grid, block, 0, s, a, g)
                            : launch_kernel(fine_bwd_dq_kernel<64>, grid, block, 0, s, a, g);
  if (e != hipSuccess) return e;
  return g.D == 128 ? launch_kernel(fine_bwd_dkdv_kernel<128>, grid, block, 0, s, a, g)
                    : launch_kernel(fine_bwd_dkdv_kernel<64>, grid, block, 0, s, a, g);
}

}  // namespace vsa
