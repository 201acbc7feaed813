// Fine stage of VSA: exact softmax attention of each 64-token query cube over
// its K selected 64-token key cubes (64x64 blocks).
//
// bf16 path (the hot loop), one workgroup = 4 waves = one query cube:
//   * wave w owns query slots 16w..16w+15; its Q fragment stays in VGPRs for
//     the whole loop;
//   * per selected key cube the K rows and the transposed V rows are staged
//     in LDS (32 KB at d=128), XOR-swizzled so the MFMA operand reads hit
//     distinct banks; the next cube's global loads are issued before the
//     current cube is multiplied, so HBM/L2 latency hides behind the MFMAs;
//   * S^T = K Q^T is computed with v_mfma_f32_16x16x32_bf16: the accumulator
//     then holds, per lane, 16 scores of ONE query row, which is exactly the
//     B-operand layout of the next product O^T += V^T P^T -- the
//     probabilities go from the softmax straight into the PV MFMAs without an
//     LDS round trip, and the O^T accumulator rows line up with the softmax
//     statistics of the same lane;
//   * online softmax in fp32 with exp2 (scale folded into one FMA); the row
//     sum is kept per lane and reduced once at the end;
//   * pad key slots of edge cubes get -inf before the max;
//   * the epilogue stages O through LDS and writes whole 16-byte chunks,
//     either in cube order or straight to raster order (fusing the inverse
//     reorder), optionally also broadcasting the coarse row of the cube to
//     every valid token (O_coarse in raster order).
// Workgroups are remapped so each XCD walks one contiguous range of
// (head, query cube) tiles, keeping that head's K/V in its own L2.
//
// fp32 path: a plain kernel, 4 threads per query row, fp32 FMA throughout.
#include "vsa_internal.h"

namespace vsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
constexpr float inv_sqrt_d() { return D == 64 ? 0.125f : 0.08838834764831845f; }

__device__ inline bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));  // RNE
}

// Halves of two words packed into one with v_perm_b32 (a's half in the low bits).
__device__ inline uint32_t lo_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ inline uint32_t hi_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Column of key kappa inside a transposed V row.  Keys 32s + 16h + 4g + r go
// to 32s + 8g + 4h + r, so the 8 keys one lane feeds to a PV MFMA k-step
// ({32s + 4g + r} and {32s + 16 + 4g + r}, r = 0..3) sit in one 16-byte run.
__device__ __host__ constexpr int vt_col(int kappa) {
  return (kappa & ~31) | (((kappa >> 2) & 3) << 3) | (((kappa >> 4) & 1) << 2) | (kappa & 3);
}

// Shared-memory tile of one key cube: K [64][D] with 16-byte chunks XOR
// swizzled by row, and V^T [D][64 (+8 pad)] with keys in vt_col order.
template <int D>
struct Tile {
  static constexpr int kKElems = 64 * D;
  static constexpr int kVtStride = 72;                 // 144 bytes: rows spread over banks
  static constexpr int kElems = kKElems + D * kVtStride;
};

// Register staging of one key cube on its way from HBM/L2 into LDS.  K rows
// are copied as 16-byte chunks; V is transposed: a thread holds 4 keys x 8
// dims and writes 8 runs of 4 keys (one per dim).
template <int D>
struct KVStage {
  static constexpr int kKC = D / 8;             // 16-byte chunks per K row
  static constexpr int kKReg = 64 * kKC / 256;  // K chunks per thread
  static constexpr int kVThreads = 2 * D;       // threads moving 4 keys x 8 dims of V
  u32x4 kreg[kKReg];
  u32x4 vreg[4];
  int tid, v_kg, v_dc;

  __device__ __forceinline__ void init(int t) {
    tid = t;
    v_kg = t % 16;   // 4-key group (consecutive lanes: consecutive groups)
    v_dc = t / 16;   // 8-dim chunk
  }
  __device__ __forceinline__ void load(const uint16_t* __restrict__ k,
                                       const uint16_t* __restrict__ v, int64_t base) {
#pragma unroll
    for (int u = 0; u < kKReg; ++u)
      kreg[u] = *reinterpret_cast<const u32x4*>(k + base + (tid + 256 * u) * 8);
    if (tid < kVThreads) {
      const uint16_t* vb = v + base + (4 * v_kg) * D + 8 * v_dc;
#pragma unroll
      for (int u = 0; u < 4; ++u) vreg[u] = *reinterpret_cast<const u32x4*>(vb + u * D);
    }
  }
  __device__ __forceinline__ void store(uint16_t* tile) const {
    uint16_t* k_lds = tile;
    uint16_t* vt_lds = tile + Tile<D>::kKElems;
#pragma unroll
    for (int u = 0; u < kKReg; ++u) {
      const int ch = tid + 256 * u, row = ch / kKC, c = ch % kKC;
      *reinterpret_cast<u32x4*>(k_lds + row * D + ((c ^ (row & (kKC - 1))) * 8)) = kreg[u];
    }
    if (tid < kVThreads) {
      // vreg[u] = V[key 4kg+u][8dc .. 8dc+7]  ->  Vt[8dc+i][vt_col(4kg) .. +3]
      const int col = vt_col(4 * v_kg);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int d0 = 8 * v_dc + 2 * h;
        const u32x2 lo = {lo_lo(vreg[0][h], vreg[1][h]), lo_lo(vreg[2][h], vreg[3][h])};
        const u32x2 hi = {hi_hi(vreg[0][h], vreg[1][h]), hi_hi(vreg[2][h], vreg[3][h])};
        *reinterpret_cast<u32x2*>(vt_lds + d0 * Tile<D>::kVtStride + col) = lo;
        *reinterpret_cast<u32x2*>(vt_lds + (d0 + 1) * Tile<D>::kVtStride + col) = hi;
      }
    }
  }
};

// Max over the 4 lanes l, l^16, l^32, l^48 that hold one query row, with the
// gfx950 cross-row swaps (VALU ops, no LDS round trip).
__device__ __forceinline__ float row_max4(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <int D, bool RASTER>
__global__ __launch_bounds__(256, 2) void fine_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx,
    uint16_t* __restrict__ o, float* __restrict__ lse, const uint16_t* __restrict__ oc,
    uint16_t* __restrict__ o_coarse, Geo g) {
  constexpr int kKC = D / 8;              // 16-byte chunks per K row
  constexpr int kKS = D / 32;             // k-steps of S^T = K Q^T
  constexpr int kDT = D / 16;             // 16-row tiles of O^T
  constexpr int kOutReg = 64 * kKC / 256; // 16-byte output chunks per thread
  constexpr int kOS = D + 8;              // padded row stride of the O staging tile
  constexpr int kVS = Tile<D>::kVtStride;
  // rescale the running output only when a row max grows by more than 2^8
  // (in exp2 units): probabilities stay <= 256, exact after normalisation
  constexpr float kTau = 8.0f;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * Tile<D>::kElems];

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bh = tile / g.C;
  const int qc = tile % g.C;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int K = g.K;
  const int32_t* __restrict__ sel = idx + static_cast<int64_t>(tile) * K;
  const float c2 = inv_sqrt_d<D>() * kLog2e;
  const float tau_raw = kTau / c2;

  // Q fragment: B operand of S^T, lane holds Q[slot 16w+li][32ks + 8lg .. +7]
  u32x4 qf[kKS];
  {
    const uint16_t* qrow = q + (bh * g.Np + static_cast<int64_t>(qc) * 64 + wave * 16 + li) * D;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
      qf[ks] = *reinterpret_cast<const u32x4*>(qrow + 32 * ks + 8 * lg);
  }

  KVStage<D> st;
  st.init(tid);

  f32x4 oacc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};   // row sums of P, by MFMA against ones
  const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};  // bf16 1.0 x 8
  float m_run = -INFINITY;

  st.load(k, v, (bh * g.Np + static_cast<int64_t>(sel[0]) * 64) * D);
  st.store(smem);
  __syncthreads();

  for (int n = 0; n < K; ++n) {
    const uint16_t* const cur = smem + (n & 1) * Tile<D>::kElems;
    const uint16_t* const k_lds = cur;
    const uint16_t* const vt_lds = cur + Tile<D>::kKElems;
    const int j = sel[n];
    const bool has_next = n + 1 < K;
    if (has_next) st.load(k, v, (bh * g.Np + static_cast<int64_t>(sel[n + 1]) * 64) * D);

    // S^T[key][q] for the 4 key tiles: lane holds S[q=li][key=16kb+4lg+r]
    // k-step outer, key tile inner: 4 independent accumulations between
    // dependent MFMAs
    f32x4 sacc[4];
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int row = 16 * kb + li;
        const int c = 4 * ks + lg;
        const u32x4 kf =
            *reinterpret_cast<const u32x4*>(k_lds + row * D + ((c ^ (row & (kKC - 1))) * 8));
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(kf), as_bf16x8(qf[ks]),
            ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[kb], 0, 0, 0);
      }
    }

    // pad key slots of an edge cube: slot 16kb + 4lg + r = (it=kb, ih=lg, iw=r)
    const CubeExt e = cube_extent(g, j);
    if (e.nt < 4 || e.nh < 4 || e.nw < 4) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kb >= e.nt || lg >= e.nh || r >= e.nw) sacc[kb][r] = -INFINITY;
    }

    // online softmax for row q = li (lanes li, li+16, li+32, li+48 share it)
    float mloc = fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3]));
#pragma unroll
    for (int kb = 1; kb < 4; ++kb)
      mloc = fmaxf(mloc, fmaxf(fmaxf(sacc[kb][0], sacc[kb][1]), fmaxf(sacc[kb][2], sacc[kb][3])));
    mloc = row_max4(mloc);
    const bool grow = mloc > m_run + tau_raw;
    if (__ballot(grow) != 0ull) {   // wave-uniform: rare after the first block
      const float m_new = grow ? mloc : m_run;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) oacc[dt] *= alpha;
      lacc *= alpha;
      m_run = m_new;
    }
    const float mb = m_run * c2;

    // P^T as B operand: k-step s covers keys 32s + 16(i/4) + 4lg + (i%4)
    u32x4 pf[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        p[i] = __builtin_amdgcn_exp2f(fmaf(sacc[2 * s + (i >> 2)][i & 3], c2, -mb));
      pf[s] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                    pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
    }
    // O^T[d][q] += V^T[d][keys] P^T[keys][q]; A lane holds Vt[16dt+li][same keys]
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ones), as_bf16x8(pf[s]), lacc,
                                                     0, 0, 0);
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
        const u32x4 a =
            *reinterpret_cast<const u32x4*>(vt_lds + (16 * dt + li) * kVS + 32 * s + 8 * lg);
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(pf[s]),
                                                           oacc[dt], 0, 0, 0);
      }
    }

    if (has_next) st.store(smem + ((n + 1) & 1) * Tile<D>::kElems);
    __syncthreads();
  }

  // ---- epilogue: l is the same in every accumulator row of lacc
  const float l = lacc[0];
  const float inv = 1.f / l;
  if (lse != nullptr && lg == 0)
    lse[bh * g.Np + static_cast<int64_t>(qc) * 64 + wave * 16 + li] = (m_run * c2 + log2f(l)) * kLn2;

  uint16_t* const o_lds = smem;  // [64][kOS]; every wave has passed the last barrier
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) {
    // lane holds O[q = 16w+li][d = 16dt + 4lg + r], r = 0..3
    const u32x2 w = {pack_bf16x2(oacc[dt][0] * inv, oacc[dt][1] * inv),
                     pack_bf16x2(oacc[dt][2] * inv, oacc[dt][3] * inv)};
    *reinterpret_cast<u32x2*>(o_lds + (wave * 16 + li) * kOS + 16 * dt + 4 * lg) = w;
  }
  __syncthreads();
  const CubeExt eq = cube_extent(g, qc);
#pragma unroll
  for (int u = 0; u < kOutReg; ++u) {
    const int ch = tid + 256 * u, row = ch / kKC, c = ch % kKC;
    const u32x4 val = *reinterpret_cast<const u32x4*>(o_lds + row * kOS + 8 * c);
    if (RASTER) {
      const int64_t tok = slot_token(g, eq, row);
      if (tok >= 0) {
        *reinterpret_cast<u32x4*>(o + (bh * g.N + tok) * D + 8 * c) = val;
        if (oc != nullptr)
          *reinterpret_cast<u32x4*>(o_coarse + (bh * g.N + tok) * D + 8 * c) =
              *reinterpret_cast<const u32x4*>(oc + (bh * g.C + qc) * D + 8 * c);
      }
    } else {
      *reinterpret_cast<u32x4*>(o + (bh * g.Np + static_cast<int64_t>(qc) * 64 + row) * D + 8 * c) = val;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32: 4 threads per query row, thread owns dims qq + 4*i; 32 keys per step.
template <int D, bool RASTER>
__global__ __launch_bounds__(256) void fine_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ idx, float* __restrict__ o, float* __restrict__ lse,
    const float* __restrict__ oc, float* __restrict__ o_coarse, Geo g) {
  constexpr int kQ = D / 4;
  constexpr int kKeys = 32;
  __shared__ float ks[kKeys * D];
  __shared__ float vs[kKeys * D];

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bh = tile / g.C;
  const int qc = tile % g.C;
  const int tid = threadIdx.x, row = tid >> 2, qq = tid & 3;
  const int K = g.K;
  const int32_t* __restrict__ sel = idx + static_cast<int64_t>(tile) * K;
  const float c2 = inv_sqrt_d<D>() * kLog2e;

  float qv[kQ], ov[kQ];
  const float* qrow = q + (bh * g.Np + static_cast<int64_t>(qc) * 64 + row) * D;
#pragma unroll
  for (int i = 0; i < kQ; ++i) {
    qv[i] = qrow[qq + 4 * i] * c2;
    ov[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int n = 0; n < K; ++n) {
    const int j = sel[n];
    const CubeExt e = cube_extent(g, j);
    for (int half = 0; half < 2; ++half) {
      __syncthreads();
      const int64_t base = (bh * g.Np + static_cast<int64_t>(j) * 64 + half * kKeys) * D;
      for (int x = tid; x < kKeys * D; x += 256) {
        ks[x] = k[base + x];
        vs[x] = v[base + x];
      }
      __syncthreads();
      float s[kKeys];
      float mloc = -INFINITY;
#pragma unroll
      for (int jj = 0; jj < kKeys; ++jj) {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < kQ; ++i) part = fmaf(qv[i], ks[jj * D + qq + 4 * i], part);
        part += __shfl_xor(part, 1);
        part += __shfl_xor(part, 2);
        const int slot = half * kKeys + jj;
        const bool valid = (slot >> 4) < e.nt && ((slot >> 2) & 3) < e.nh && (slot & 3) < e.nw;
        s[jj] = valid ? part : -INFINITY;
        mloc = fmaxf(mloc, s[jj]);
      }
      const float m_new = fmaxf(m, mloc);   // slot 0 of every cube is valid
      const float alpha = exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int i = 0; i < kQ; ++i) ov[i] *= alpha;
#pragma unroll
      for (int jj = 0; jj < kKeys; ++jj) {
        const float pj = exp2f(s[jj] - m_new);
        l += pj;
#pragma unroll
        for (int i = 0; i < kQ; ++i) ov[i] = fmaf(pj, vs[jj * D + qq + 4 * i], ov[i]);
      }
      m = m_new;
    }
  }

  const float inv = 1.f / l;
  if (lse != nullptr && qq == 0)
    lse[bh * g.Np + static_cast<int64_t>(qc) * 64 + row] = (m + log2f(l)) * kLn2;
  if (RASTER) {
    const CubeExt eq = cube_extent(g, qc);
    const int64_t tok = slot_token(g, eq, row);
    if (tok >= 0) {
      float* orow = o + (bh * g.N + tok) * D;
#pragma unroll
      for (int i = 0; i < kQ; ++i) orow[qq + 4 * i] = ov[i] * inv;
      if (oc != nullptr) {
        const float* crow = oc + (bh * g.C + qc) * D;
        float* corow = o_coarse + (bh * g.N + tok) * D;
#pragma unroll
        for (int i = 0; i < kQ; ++i) corow[qq + 4 * i] = crow[qq + 4 * i];
      }
    }
  } else {
    float* orow = o + (bh * g.Np + static_cast<int64_t>(qc) * 64 + row) * D;
#pragma unroll
    for (int i = 0; i < kQ; ++i) orow[qq + 4 * i] = ov[i] * inv;
  }
}

template <int D, bool RASTER>
hipError_t launch_typed(const Geo& g, int dtype, const void* q, const void* k, const void* v,
                        const int32_t* idx, void* o, float* lse, const void* oc,
                        void* o_coarse, hipStream_t s) {
  const dim3 grid(g.B * g.H * g.C), block(256);
  if (dtype == 1)
    return launch_kernel(fine_fwd_bf16_kernel<D, RASTER>, grid, block, 0, s,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                         static_cast<const uint16_t*>(v), idx, static_cast<uint16_t*>(o), lse,
                         static_cast<const uint16_t*>(oc), static_cast<uint16_t*>(o_coarse), g);
  return launch_kernel(fine_fwd_f32_kernel<D, RASTER>, grid, block, 0, s,
                       static_cast<const float*>(q), static_cast<const float*>(k),
                       static_cast<const float*>(v), idx, static_cast<float*>(o), lse,
                       static_cast<const float*>(oc), static_cast<float*>(o_coarse), g);
}

}  // namespace

hipError_t launch_fine(const Geo& g, int dtype, const void* q, const void* k, const void* v,
                       const int32_t* idx, void* o, float* lse, bool raster_out,
                       const void* oc, void* o_coarse, hipStream_t s) {
  if (g.D == 128)
    return raster_out ? launch_typed<128, true>(g, dtype, q, k, v, idx, o, lse, oc, o_coarse, s)
                      : launch_typed<128, false>(g, dtype, q, k, v, idx, o, lse, oc, o_coarse, s);
  return raster_out ? launch_typed<64, true>(g, dtype, q, k, v, idx, o, lse, oc, o_coarse, s)
                    : launch_typed<64, false>(g, dtype, q, k, v, idx, o, lse, oc, o_coarse, s);
}

}  // namespace vsa
