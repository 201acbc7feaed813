// Dense flash attention over every key cube of a head (no index list), bf16,
// cube-order tensors: the baseline the sparse fine stage is measured against.
// It is built with the compiler's default instruction scheduling; the sparse
// kernel's source is built with the memory-clause scheduler, which is slower
// here.
#include "attn_tile.h"

namespace vsa {
namespace {

// Dense flash attention over every key cube (no index list): the baseline
// the sparse stage is measured against.  One workgroup of 4 waves owns two
// consecutive query cubes of a head, 128 query rows; wave w owns slots
// 32(w%2)..+31 of cube 2t + w/2 as two 16-row blocks.  All four waves share
// one stream of K and V, taken half a key cube (32 keys) per step, so every
// staged byte serves 128 query rows and every K or V fragment read from LDS
// feeds the MFMAs of two row blocks.  The step is that of the sparse kernel:
// DMA into XOR-swizzled LDS, S^T = K Q^T, transposed V reads, lazy running
// max, row sums from an MFMA against ones; pad keys are masked by the key
// cube's extent.  q, k, v and o are cube order [B,H,Np,D].
template <int D>
__global__ __launch_bounds__(256, 2) void dense_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse, Geo g) {
  using Tl = HalfTile<D>;
  constexpr int kKC = Tl::kKC;
  constexpr int kKS = D / 32;              // k-steps of S^T = K Q^T
  constexpr int kDT = D / 16;              // 16-row tiles of O^T
  constexpr int kT = Tl::kElems;
  constexpr int kOS = D + 8;               // padded row stride of the O staging tile
  constexpr int kOutReg = 128 * kKC / 256; // 16-byte output chunks per thread
  constexpr float kTau = 8.0f;             // lazy rescale threshold (exp2 units)
  constexpr int kSmem = (4 * kT > 128 * kOS) ? 4 * kT : 128 * kOS;
  __shared__ __attribute__((aligned(16))) uint16_t smem[kSmem];   // K ring (2), V ring (2) | O
  uint16_t* const kring = smem;
  uint16_t* const vring = smem + 2 * kT;

  const int pairs = (g.C + 1) / 2;                       // query-cube pairs per head
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bh = tile / pairs;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int qc = 2 * (tile % pairs) + (wave >> 1);       // this wave's query cube
  const int C = g.C, steps = 2 * C;
  const float c2 = inv_sqrt_d<D>() * kLog2e;
  const int64_t head0 = bh * g.Np * D;
  const uint32_t head_bytes = static_cast<uint32_t>(g.Np * D * 2);
  const __amdgpu_buffer_rsrc_t krs = head_rsrc(k + head0, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc(v + head0, head_bytes);

  // DMA byte offsets (from a half tile's first row) of this thread's chunks:
  // chunk P = 256u + tid is row P / kKC of the half tile, stored swizzled
  uint32_t koff[Tl::kDma], voff[Tl::kDma];
#pragma unroll
  for (int u = 0; u < Tl::kDma; ++u) {
    const int P = u * 256 + tid;
    const int r = P / kKC, c = P % kKC;
    koff[u] = static_cast<uint32_t>(r * D * 2 + (c ^ FineTile<D>::ksw(r)) * 16);
    voff[u] = static_cast<uint32_t>(r * D * 2 + (c ^ FineTile<D>::vsw(r)) * 16);
  }
  // step n: key cube n/2, half n%2 (32 rows), contiguous in cube order
  auto stage = [&](const __amdgpu_buffer_rsrc_t& rs, const uint32_t* off, int n, uint16_t* slot) {
    dma_half<D>(rs, static_cast<uint32_t>(n * 32 * D * 2), off, slot, wave);
  };

  // Q fragments (a wave past the last cube of an odd C reads cube C-1 and
  // writes nothing)
  const bool real = qc < C;
  u32x4 qf[2][kKS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = min(qc, C - 1) * 64 + 32 * (wave & 1) + 16 * qb + li;
    const uint16_t* qrow = q + head0 + static_cast<int64_t>(row) * D;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
      qf[qb][ks] = *reinterpret_cast<const u32x4*>(qrow + 32 * ks + 8 * lg);
  }
  int kro[kKS], vtr[kDT];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) kro[ks] = li * D + (((4 * ks + lg) ^ FineTile<D>::ksw(li)) * 8);
  {
    const int r = 4 * lg + (li >> 2);
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
      vtr[dt] = r * D + (((2 * dt + ((li & 3) >> 1)) ^ FineTile<D>::vsw(r)) * 8) + (li & 1) * 4;
  }
  f32x4 oacc[2][kDT];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) oacc[qb][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 lacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};

  // extents of key cubes first..first+63, one per lane
  int ext_lanes;
  auto load_ext = [&](int first) {
    const int c = first + lane;
    ext_lanes = kFullExt;
    if (c < C) {
      const CubeExt e = cube_extent(g, c);
      ext_lanes = e.nt | (e.nh << 3) | (e.nw << 6);
    }
  };
  load_ext(0);
  auto key_ext = [&](int m) { return __builtin_amdgcn_readlane(ext_lanes, m & 63); };

  stage(krs, koff, 0, kring);
  stage(vrs, voff, 0, vring);
  stage(krs, koff, 1, kring + kT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const int ext0 = key_ext(0);
  int hw_cur = ext0 >> 3;
  f32x4 bias = hw_bias(ext0, lg);
  f32x4 tcur[2][2];
  float mb[2];
  float mbk[2][2];
  score_half<D, 2>(kring, kro, qf, bias, tcur);
  {
    const bool v1 = (ext0 & 7) > 1;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      tcur[qb][0] = tcur[qb][0] * c2;
      tcur[qb][1] = v1 ? tcur[qb][1] * c2 : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      mb[qb] = row_max8(tcur[qb]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) tcur[qb][kb] = tcur[qb][kb] - mb[qb];
    }
  }

  auto step = [&](auto p0c, int n) {
    constexpr int P0 = decltype(p0c)::value, P1 = P0 ^ 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int m1 = (n + 1) >> 1;
    const int ext = key_ext(m1);
    stage(vrs, voff, n + 1, vring + P1 * kT);
    if (n + 2 < steps) {
      if (P0 == 0 && (((n + 2) >> 1) & 63) == 0) load_ext((n + 2) >> 1);
      stage(krs, koff, n + 2, kring + P0 * kT);
    }
    if (P0 == 1 && (ext >> 3) != hw_cur) {
      hw_cur = ext >> 3;
      bias = hw_bias(ext, lg);
    }
    const int nt = ext & 7;
    const float o0 = 2 * P1 < nt ? 0.f : -INFINITY, o1 = 2 * P1 + 1 < nt ? 0.f : -INFINITY;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      mbk[qb][0] = o0 - mb[qb];
      mbk[qb][1] = o1 - mb[qb];
    }
    f32x4 tnext[2][2];
    score_half<D, 2>(kring + P1 * kT, kro, qf, bias, tnext);
    u32x4 pf[2];
    probabilities_half<2>(tcur, pf);
    pv_half<D, 2>(vring + P0 * kT, vtr, pf, oacc, lacc);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) tnext[qb][kb][r] = fmaf(tnext[qb][kb][r], c2, mbk[qb][kb]);
    if (__ballot(fmaxf(lane_max8(tnext[0]), lane_max8(tnext[1])) > kTau) != 0ull) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float mt = row_max8(tnext[qb]);
        const float delta = mt > kTau ? mt : 0.f;
        const float alpha = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) oacc[qb][dt] *= alpha;
        lacc[qb] *= alpha;
        mb[qb] += delta;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) tnext[qb][kb] = tnext[qb][kb] - delta;
      }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) tcur[qb][kb] = tnext[qb][kb];
  };
  for (int n = 0; n < steps - 1; n += 2) {
    step(std::integral_constant<int, 0>{}, n);
    if (n + 2 >= steps) break;
    step(std::integral_constant<int, 1>{}, n + 1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  {
    u32x4 pf[2];
    probabilities_half<2>(tcur, pf);
    pv_half<D, 2>(vring + kT, vtr, pf, oacc, lacc);   // the last step is a second half
  }
  __syncthreads();

  uint16_t* const o_lds = smem;  // [128][kOS]
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = lacc[qb][0];
    const float inv = 1.f / l;
    const int slot = 32 * (wave & 1) + 16 * qb + li;
    if (lse != nullptr && lg == 0 && real)
      lse[bh * g.Np + static_cast<int64_t>(qc) * 64 + slot] = (mb[qb] + log2f(l)) * kLn2;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) {
      const u32x2 w = {pack_bf16x2(oacc[qb][dt][0] * inv, oacc[qb][dt][1] * inv),
                       pack_bf16x2(oacc[qb][dt][2] * inv, oacc[qb][dt][3] * inv)};
      *reinterpret_cast<u32x2*>(o_lds + (64 * (wave >> 1) + slot) * kOS + 16 * dt + 4 * lg) = w;
    }
  }
  __syncthreads();
  const int64_t orow0 = bh * g.Np + static_cast<int64_t>(2 * (tile % pairs)) * 64;
#pragma unroll
  for (int u = 0; u < kOutReg; ++u) {
    const int ch = tid + 256 * u, row = ch / kKC, c = ch % kKC;
    if (2 * (tile % pairs) + (row >> 6) < C)
      *reinterpret_cast<u32x4*>(o + (orow0 + row) * D + 8 * c) =
          *reinterpret_cast<const u32x4*>(o_lds + row * kOS + 8 * c);
  }
}

}  // namespace

hipError_t launch_dense(const Geo& g, const void* q, const void* k, const void* v, void* o,
                        float* lse, hipStream_t s) {
  const dim3 grid(g.B * g.H * ((g.C + 1) / 2)), block(256);
  auto qq = static_cast<const uint16_t*>(q), kk = static_cast<const uint16_t*>(k),
       vv = static_cast<const uint16_t*>(v);
  auto oo = static_cast<uint16_t*>(o);
  if (g.D == 128) return launch_kernel(dense_fwd_bf16_kernel<128>, grid, block, 0, s, qq, kk, vv, oo, lse, g);
  return launch_kernel(dense_fwd_bf16_kernel<64>, grid, block, 0, s, qq, kk, vv, oo, lse, g);
}

}  // namespace vsa
