// Fine stage of VSA: exact softmax attention of each 64-token query cube over
// its K selected 64-token key cubes (64x64 blocks).
//
// bf16 path (the hot loop), one workgroup = 4 waves = one query cube; each
// wave owns 16 query slots (a time slice or an h-row of the cube) and keeps
// their Q fragment in VGPRs; a wave whose slots are all pads computes nothing.
//   * Gather: q, k, v are read either in cube order (64 rows per cube) or
//     straight from raster order, where slot (it, ih, iw) of a cube is row
//     base(cube) + (it*Hh + ih)*Ww + iw, so no reordered copy is needed.
//   * Steps of half a key cube: a key cube is taken as two halves of 32
//     keys (time slices 0-1 and 2-3), one half per step.  The K and V rings
//     then hold two half tiles each, 32 KB at D = 128, and the step keeps
//     only 32 scores per query row in registers (<= 168 VGPRs), so three
//     workgroups share a CU instead of two: measured, the third workgroup
//     hides the start and end of each tile (idx load, first DMA, O stores)
//     and more than pays for the second barrier per key cube.
//   * Staging: the K rows and V rows of a half go from HBM/L2 straight into
//     LDS with buffer_load_dwordx4 ... lds (no VGPRs; the per-lane offsets
//     stay in registers and only a scalar row offset changes from half to
//     half, so staging costs no VALU).  Each lane's source chunk is chosen
//     so that LDS holds the tiles XOR-swizzled for the reads below; K runs
//     one half ahead of V.  Pad slots of a raster edge cube read their own
//     raster address (a neighbouring token, or zeros past the head's rows):
//     finite values, masked to probability 0.
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: the accumulator then holds,
//     per lane, 16 scores of ONE query row, which is the B-operand layout of
//     O^T += V^T P^T, so probabilities go from the softmax straight into the
//     PV MFMAs.  The V^T operand comes from row-major V by gfx950 transposed
//     LDS reads (ds_read_b64_tr_b16).
//   * Pad key slots: one accumulator init (0 / -inf) masks the (ih, iw) part
//     for every key block; blocks past the cube's t extent get a -inf offset
//     in the exp2 argument.  Extents come from a per-lane table, one
//     v_readlane per key cube, and the (ih, iw) mask changes only when the
//     extent does.
//   * Software pipeline per wave: while the MFMAs of S(j+1) run, the VALU
//     evaluates exp2 of half j; while PV(j) runs, it scales S(j+1) into exp2
//     units (t = s log2(e)/sqrt(d) - m).  The running max m is raised
//     lazily (only when a row exceeds it by 2^8), so probabilities stay
//     <= 256; the common step checks each lane's own maximum against that
//     bound and needs neither the cross-lane row max nor a rescale.
//   * Row sums come from one extra MFMA per half against a ones operand.
//   * The epilogue stages O through LDS and writes whole 16-byte chunks,
//     either in cube order or straight to raster order (fusing the inverse
//     reorder), optionally also broadcasting the coarse row of the cube to
//     every valid token (O_coarse in raster order).
// Workgroups are remapped so each XCD walks one contiguous range of
// (head, query cube) tiles, keeping that head's K/V in its own L2.
// This source is compiled with LLVM's memory-clause scheduling strategy
// (block_sparse_attention_cube_amd/build.py): under the 168-VGPR budget the
// default strategy serialises the K-fragment LDS reads behind the MFMAs.
#include <type_traits>

#include "attn_tile.h"

namespace vsa {
namespace {

// Extent and first row of the key cubes sel[first .. first+63], one per
// lane, so that a step reads them with one v_readlane each.
template <bool RASTER>
__device__ __forceinline__ void lane_keys(const Geo& g, const int32_t* __restrict__ sel, int first,
                                          int K, int lane, int& ext, int& row) {
  ext = kFullExt;
  row = 0;
  const int m = first + lane;
  if (m < K) {
    const int c = sel[m];
    const CubeExt e = cube_extent(g, c);
    ext = e.nt | (e.nh << 3) | (e.nw << 6);
    row = cube_row<RASTER>(g, e, c);
  }
}

// RASTER: q, k, v are raster [B,H,N,D] and o, o_coarse are raster;
// otherwise q, k, v and o are cube order [B,H,Np,D].
// HROWS: wave w owns the 16 query slots of the cube's h-row ih = w (slot
// 16 it + 4 w + iw) instead of its time slice it = w (slots 16w..16w+15); a
// wave whose row or slice lies past the cube's extent holds only pad slots
// and computes nothing.  The launcher takes the mapping that idles more
// waves on the grid at hand.
// EMPTY_HALVES: the grid's last cube layer is at most two time slices deep
// (T % 4 in {1, 2}), so its key cubes have an empty second half, whose
// staging and work are skipped; the launcher sets it from the grid, and
// without it the step carries no test for the case.
template <int D, bool RASTER, bool HROWS, bool EMPTY_HALVES>
__global__ __launch_bounds__(256, 3) void fine_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx,
    uint16_t* __restrict__ o, float* __restrict__ lse, const uint16_t* __restrict__ oc,
    uint16_t* __restrict__ o_coarse, Geo g) {
  using Tl = FineTile<D>;
  using Hl = HalfTile<D>;
  constexpr int kKC = Tl::kKC;
  constexpr int kKS = D / 32;              // k-steps of S^T = K Q^T
  constexpr int kDT = D / 16;              // 16-row tiles of O^T
  constexpr int kH = Hl::kElems;           // elements of a half tile
  constexpr int kOutReg = 64 * kKC / 256;  // 16-byte output chunks per thread
  constexpr int kOS = D + 8;               // padded row stride of the O staging tile
  constexpr float kTau = 8.0f;             // lazy rescale threshold (exp2 units)
  static_assert(64 * kOS <= 4 * kH, "the O staging tile fits in the rings");
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * kH];   // K ring (2), V ring (2)
  uint16_t* const kring = smem;
  uint16_t* const vring = smem + 2 * kH;

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bh = tile / g.C;
  const int qc = tile % g.C;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int K = g.K;
  const int32_t* __restrict__ sel = idx + static_cast<int64_t>(tile) * K;
  const float c2 = inv_sqrt_d<D>() * kLog2e;
  const int64_t head0 = bh * (RASTER ? g.N : g.Np) * D;   // element offset of this head's rows
  const uint32_t head_bytes = static_cast<uint32_t>((RASTER ? g.N : g.Np) * D * 2);
  const __amdgpu_buffer_rsrc_t krs = head_rsrc(k + head0, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc(v + head0, head_bytes);

  // DMA byte offsets (from the cube's first row) of this thread's chunks of
  // the first half (time slices 0, 1); the second half starts half_rows
  // rows further on.  A pad slot of a raster edge cube reads its own raster
  // address all the same: a token of a neighbouring row or frame, or past
  // the head's rows, where the buffer resource returns zeros.  Either way a
  // finite value whose probability the masks below make exactly 0.
  uint32_t koff[Hl::kDma], voff[Hl::kDma];
#pragma unroll
  for (int u = 0; u < Hl::kDma; ++u) {
    const int P = u * 256 + tid;
    const int r = P / kKC, c = P % kKC;
    int it, ih, iw;
    dma_slot<D>(u, wave, lane, it, ih, iw);
    const uint32_t rowoff = static_cast<uint32_t>(slot_row<RASTER>(g, it, ih, iw) * D) * 2u;
    koff[u] = rowoff + (c ^ Tl::ksw(r)) * 16;
    voff[u] = rowoff + (c ^ Tl::vsw(r)) * 16;
  }
  const int half_rows = slot_row<RASTER>(g, 2, 0, 0);
  // stage half h of the K or V tile of a key cube (first row `row`)
  auto stage = [&](const __amdgpu_buffer_rsrc_t& rs, const uint32_t* off, int row, int h,
                   uint16_t* slot) {
    dma_half<D>(rs, static_cast<uint32_t>(row + h * half_rows) * (D * 2), off, slot, wave);
  };

  // Q fragment: B operand of S^T, lane holds Q[slot 16w+li][32ks + 8lg .. +7]
  u32x4 qf[1][kKS];
  const CubeExt eq = cube_extent(g, qc);
  // wave w holds time slice w (or h-row w) of the query cube: past the
  // cube's extent its 16 slots are all pads and it computes nothing (it
  // still stages its share of the tiles and meets every barrier).  Lane li
  // serves query slot qslot.
  const bool active = wave < (HROWS ? eq.nh : eq.nt);
  const int qslot = HROWS ? 16 * (li >> 2) + 4 * wave + (li & 3) : 16 * wave + li;
  {
    const int it = qslot >> 4, ih = (qslot >> 2) & 3, iw = li & 3;
    const bool valid = !RASTER || (it < eq.nt && ih < eq.nh && iw < eq.nw);
    const int row = cube_row<RASTER>(g, eq, qc) + (valid ? slot_row<RASTER>(g, it, ih, iw) : 0);
    const uint16_t* qrow = q + head0 + static_cast<int64_t>(row) * D;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
      qf[0][ks] = *reinterpret_cast<const u32x4*>(qrow + 32 * ks + 8 * lg);
  }
  // per-lane LDS element offsets of the operand reads (loop invariant)
  int kro[kKS], vtr[kDT];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) kro[ks] = li * D + (((4 * ks + lg) ^ Tl::ksw(li)) * 8);
  {
    const int r = 4 * lg + (li >> 2);        // V row of the half's first key block this lane supplies
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
      vtr[dt] = r * D + (((2 * dt + ((li & 3) >> 1)) ^ Tl::vsw(r)) * 8) + (li & 1) * 4;
  }

  f32x4 oacc[1][kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) oacc[0][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 lacc[1] = {{0.f, 0.f, 0.f, 0.f}};

  // key cube extents and first rows, 64 cubes per lane vector
  int ext_lanes, row_lanes;
  lane_keys<RASTER>(g, sel, 0, K, lane, ext_lanes, row_lanes);
  auto key_ext = [&](int n) { return __builtin_amdgcn_readlane(ext_lanes, n & 63); };
  auto key_row = [&](int n) { return __builtin_amdgcn_readlane(row_lanes, n & 63); };

  // With EMPTY_HALVES, a key cube whose t extent is at most 2 (the last
  // cube layer) has an empty second half: its K and V halves are not staged
  // and the steps next to it do only the other half's work.

  // prologue: both K halves (the second unless empty) and the first V half
  // of key cube 0 in flight together; S of the first half and its row max
  const int ext0 = key_ext(0), row0 = key_row(0);
  stage(krs, koff, row0, 0, kring);
  stage(vrs, voff, row0, 0, vring);
  if (!EMPTY_HALVES || (ext0 & 7) > 2) stage(krs, koff, row0, 1, kring + kH);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // the (ih, iw) mask follows the key cube's extent and is rebuilt only when
  // it changes; nt_cur is the t extent of the cube whose halves are in play
  int hw_cur = ext0 >> 3, nt_cur = ext0 & 7;
  f32x4 bias = hw_bias(ext0, lg);
  f32x4 tcur[1][2];
  // S(0) runs on every wave, also on one past the t extent (its Q rows are
  // redirected to real ones), so that the Q loads are consumed on every path
  // before the loop: the compiler then places no wait for them inside it,
  // where its count of outstanding loads would not include the tile DMA
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) asm volatile("" :: "v"(qf[0][ks]));   // Q has landed, every path
  score_half<D, 1>(kring, kro, qf, bias, tcur);
  // time slice 0 always holds a valid key; slice 1 may lie past the extent
  tcur[0][0] = tcur[0][0] * c2;
  tcur[0][1] = nt_cur > 1 ? tcur[0][1] * c2 : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  float mb = row_max8(tcur[0]);   // running row max, exp2 units
  tcur[0][0] = tcur[0][0] - mb;
  tcur[0][1] = tcur[0][1] - mb;

  // The work of a step: S of half j+1 from K slot ks (DO_S), exp2 and PV of
  // half j from V slot vs (DO_PV); a step next to an empty half does one of
  // the two, in code of its own so that the full step keeps its schedule.
  auto work = [&](auto do_s, auto do_pv, const uint16_t* ks, const uint16_t* vs, float off0,
                  float off1) {
    constexpr bool DO_S = decltype(do_s)::value, DO_PV = decltype(do_pv)::value;
    f32x4 tnext[1][2];
    if (DO_S) score_half<D, 1>(ks, kro, qf, bias, tnext);
    if (DO_PV) {
      u32x4 pf[1];
      probabilities_half<1>(tcur, pf);
      pv_half<D, 1>(vs, vtr, pf, oacc, lacc);
    }
    if (!DO_S) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      tnext[0][0][r] = fmaf(tnext[0][0][r], c2, off0);
      tnext[0][1][r] = fmaf(tnext[0][1][r], c2, off1);
    }
    // Every value of the wave within 2^tau of the running max (the common
    // case) needs no row max at all: the cross-lane reduction and the rescale
    // run only when some lane exceeds it.  Wave-uniform branch.
    if (__ballot(lane_max8(tnext[0]) > kTau) != 0ull) {
      const float mt = row_max8(tnext[0]);
      const float delta = mt > kTau ? mt : 0.f;
      const float alpha = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) oacc[0][dt] *= alpha;
      lacc[0] *= alpha;
      mb += delta;
      tnext[0][0] = tnext[0][0] - delta;
      tnext[0][1] = tnext[0][1] - delta;
    }
    tcur[0][0] = tnext[0][0];
    tcur[0][1] = tnext[0][1];
  };
  using T = std::true_type;
  using F = std::false_type;
  // One step per half key cube, j = 2n + H: the K half j+1 and the V half j
  // have landed.  S of half j+1 runs on the matrix cores while exp2 of half
  // j runs on the VALU, then PV of half j while S of half j+1 is scaled into
  // exp2 units.  Half j sits in ring slot H of both rings, so every LDS
  // address is a register plus an immediate offset.
  auto step = [&](auto hc, int n) {
    constexpr int H = decltype(hc)::value;
    // the slots of K half j and V half j-1 are free for every wave
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // nt_cur: t extent of cube n (H = 0), of cube n + 1 (H = 1, below)
    const bool full_n = !EMPTY_HALVES || nt_cur > 2;   // cube n has a second half (H = 0)
    int ext = 0;
    if (H == 0) {
      // half j+1 is the second half of cube n; the next K half to stage is
      // the first of cube n + 1
      if (full_n) stage(vrs, voff, key_row(n), 1, vring + kH);
      if (n + 1 < K) {
        if (((n + 1) & 63) == 0) lane_keys<RASTER>(g, sel, n + 1, K, lane, ext_lanes, row_lanes);
        stage(krs, koff, key_row(n + 1), 0, kring);
      }
    } else {
      // half j+1 is the first half of cube n + 1 (present: the loop ends
      // after the first half of the last cube)
      const int row = key_row(n + 1);
      ext = key_ext(n + 1);
      stage(vrs, voff, row, 0, vring);
      if (!EMPTY_HALVES || (ext & 7) > 2) stage(krs, koff, row, 1, kring + kH);
    }
    if (!active) {
      if (H == 1) nt_cur = ext & 7;
      return;
    }
    if (H == 0) {
      // exp2 offsets of the two key blocks of the second half (time slices
      // 2 and 3): -mb, or -inf past the cube's t extent
      if (full_n) work(T{}, T{}, kring + kH, vring, -mb, nt_cur > 3 ? -mb : -INFINITY);
      else work(F{}, T{}, kring + kH, vring, 0.f, 0.f);
    } else {
      if ((ext >> 3) != hw_cur) {
        hw_cur = ext >> 3;
        bias = hw_bias(ext, lg);
      }
      nt_cur = ext & 7;
      // time slices 0 and 1 of cube n + 1: slice 0 always holds a valid key
      const float off1 = nt_cur > 1 ? -mb : -INFINITY;
      if (full_n) work(T{}, T{}, kring, vring + kH, -mb, off1);
      else work(T{}, F{}, kring, vring + kH, -mb, off1);
    }
  };
  for (int n = 0;; ++n) {
    step(std::integral_constant<int, 0>{}, n);
    if (n + 1 >= K) break;
    step(std::integral_constant<int, 1>{}, n);
  }
  // the second V half of the last cube has landed (if it has one)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (active && (!EMPTY_HALVES || nt_cur > 2)) {
    u32x4 pf[1];
    probabilities_half<1>(tcur, pf);
    pv_half<D, 1>(vring + kH, vtr, pf, oacc, lacc);
  }
  __syncthreads();   // every wave is done with the rings: reuse them for O

  // ---- epilogue: l is the same in every accumulator row of lacc; a wave
  // past the t extent writes zeros (pad rows)
  const float l = lacc[0][0];
  const float inv = active ? 1.f / l : 0.f;
  if (lse != nullptr && lg == 0)
    lse[bh * g.Np + static_cast<int64_t>(qc) * 64 + qslot] =
        active ? (mb + log2f(l)) * kLn2 : 0.f;

  uint16_t* const o_lds = smem;  // [64][kOS]
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) {
    // lane holds O[q = qslot][d = 16dt + 4lg + r], r = 0..3
    const u32x2 w = {pack_bf16x2(oacc[0][dt][0] * inv, oacc[0][dt][1] * inv),
                     pack_bf16x2(oacc[0][dt][2] * inv, oacc[0][dt][3] * inv)};
    *reinterpret_cast<u32x2*>(o_lds + qslot * kOS + 16 * dt + 4 * lg) = w;
  }
  __syncthreads();
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
// fp32: 4 threads per query row, thread qq owns the contiguous dims
// qq*D/4 .. qq*D/4 + D/4 - 1; 32 keys per step, read from LDS 16 bytes at a
// time and four keys per batch so that the reads of a batch overlap.  Row
// dot products are summed over the row's 4 lanes with DPP quad permutes;
// exponentials use the hardware v_exp_f32 (about 1 ulp).
template <int D, bool RASTER>
__global__ __launch_bounds__(256) void fine_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ idx, float* __restrict__ o, float* __restrict__ lse,
    const float* __restrict__ oc, float* __restrict__ o_coarse, Geo g) {
  constexpr int kQ = D / 4;       // dims per thread
  constexpr int kQ4 = kQ / 4;     // float4 per thread
  constexpr int kKeys = 32;
  constexpr int kBatch = 4;
  __shared__ __attribute__((aligned(16))) float ks[kKeys * D];
  __shared__ __attribute__((aligned(16))) float vs[kKeys * D];

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bh = tile / g.C;
  const int qc = tile % g.C;
  const int tid = threadIdx.x, row = tid >> 2, qq = tid & 3;
  const int K = g.K;
  const int32_t* __restrict__ sel = idx + static_cast<int64_t>(tile) * K;
  const float c2 = inv_sqrt_d<D>() * kLog2e;
  const int d0 = qq * kQ;

  float4 qv[kQ4], ov[kQ4];
  const float* qrow = q + (bh * g.Np + static_cast<int64_t>(qc) * 64 + row) * D + d0;
#pragma unroll
  for (int i = 0; i < kQ4; ++i) {
    const float4 x = reinterpret_cast<const float4*>(qrow)[i];
    qv[i] = make_float4(x.x * c2, x.y * c2, x.z * c2, x.w * c2);
    ov[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float m = -INFINITY, l = 0.f;
  auto quad_sum = [](float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));
    return x;
  };

  for (int n = 0; n < K; ++n) {
    const int j = sel[n];
    const CubeExt e = cube_extent(g, j);
    for (int half = 0; half < 2; ++half) {
      __syncthreads();
      const int64_t base = (bh * g.Np + static_cast<int64_t>(j) * 64 + half * kKeys) * D;
#pragma unroll
      for (int x = tid; x < kKeys * D / 4; x += 256) {
        reinterpret_cast<float4*>(ks)[x] = reinterpret_cast<const float4*>(k + base)[x];
        reinterpret_cast<float4*>(vs)[x] = reinterpret_cast<const float4*>(v + base)[x];
      }
      __syncthreads();
      float s[kKeys];
      float mloc = -INFINITY;
#pragma unroll
      for (int j0 = 0; j0 < kKeys; j0 += kBatch) {
        float4 kr[kBatch][kQ4];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
#pragma unroll
          for (int i = 0; i < kQ4; ++i)
            kr[u][i] = *reinterpret_cast<const float4*>(ks + (j0 + u) * D + d0 + 4 * i);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          float part = 0.f;
#pragma unroll
          for (int i = 0; i < kQ4; ++i) {
            part = fmaf(qv[i].x, kr[u][i].x, part);
            part = fmaf(qv[i].y, kr[u][i].y, part);
            part = fmaf(qv[i].z, kr[u][i].z, part);
            part = fmaf(qv[i].w, kr[u][i].w, part);
          }
          part = quad_sum(part);
          const int slot = half * kKeys + j0 + u;
          const bool valid = (slot >> 4) < e.nt && ((slot >> 2) & 3) < e.nh && (slot & 3) < e.nw;
          s[j0 + u] = valid ? part : -INFINITY;
          mloc = fmaxf(mloc, s[j0 + u]);
        }
      }
      const float m_new = fmaxf(m, mloc);   // slot 0 of every cube is valid
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int i = 0; i < kQ4; ++i)
        ov[i] = make_float4(ov[i].x * alpha, ov[i].y * alpha, ov[i].z * alpha, ov[i].w * alpha);
#pragma unroll
      for (int j0 = 0; j0 < kKeys; j0 += kBatch) {
        float4 vr[kBatch][kQ4];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
#pragma unroll
          for (int i = 0; i < kQ4; ++i)
            vr[u][i] = *reinterpret_cast<const float4*>(vs + (j0 + u) * D + d0 + 4 * i);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const float pj = __builtin_amdgcn_exp2f(s[j0 + u] - m_new);
          l += pj;
#pragma unroll
          for (int i = 0; i < kQ4; ++i) {
            ov[i].x = fmaf(pj, vr[u][i].x, ov[i].x);
            ov[i].y = fmaf(pj, vr[u][i].y, ov[i].y);
            ov[i].z = fmaf(pj, vr[u][i].z, ov[i].z);
            ov[i].w = fmaf(pj, vr[u][i].w, ov[i].w);
          }
        }
      }
      m = m_new;
    }
  }

  const float inv = 1.f / l;
  if (lse != nullptr && qq == 0)
    lse[bh * g.Np + static_cast<int64_t>(qc) * 64 + row] = (m + log2f(l)) * kLn2;
  auto put = [&](float* dst) {
#pragma unroll
    for (int i = 0; i < kQ4; ++i)
      reinterpret_cast<float4*>(dst + d0)[i] =
          make_float4(ov[i].x * inv, ov[i].y * inv, ov[i].z * inv, ov[i].w * inv);
  };
  if (RASTER) {
    const CubeExt eq = cube_extent(g, qc);
    const int64_t tok = slot_token(g, eq, row);
    if (tok >= 0) {
      put(o + (bh * g.N + tok) * D);
      if (oc != nullptr) {
        const float4* crow = reinterpret_cast<const float4*>(oc + (bh * g.C + qc) * D + d0);
        float4* corow = reinterpret_cast<float4*>(o_coarse + (bh * g.N + tok) * D + d0);
#pragma unroll
        for (int i = 0; i < kQ4; ++i) corow[i] = crow[i];
      }
    }
  } else {
    put(o + (bh * g.Np + static_cast<int64_t>(qc) * 64 + row) * D);
  }
}

template <int D, bool RASTER>
hipError_t launch_typed(const Geo& g, int dtype, const void* q, const void* k, const void* v,
                        const int32_t* idx, void* o, float* lse, const void* oc,
                        void* o_coarse, hipStream_t s) {
  const dim3 grid(g.B * g.H * g.C), block(256);
  if (dtype == 1) {
    const bool hrows = waves_hold_h_rows(g), empty_halves = g.T % 4 == 1 || g.T % 4 == 2;
    auto kern = hrows ? (empty_halves ? fine_fwd_bf16_kernel<D, RASTER, true, true>
                                      : fine_fwd_bf16_kernel<D, RASTER, true, false>)
                      : (empty_halves ? fine_fwd_bf16_kernel<D, RASTER, false, true>
                                      : fine_fwd_bf16_kernel<D, RASTER, false, false>);
    return launch_kernel(kern, grid, block, 0, s,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                         static_cast<const uint16_t*>(v), idx, static_cast<uint16_t*>(o), lse,
                         static_cast<const uint16_t*>(oc), static_cast<uint16_t*>(o_coarse), g);
  }
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
