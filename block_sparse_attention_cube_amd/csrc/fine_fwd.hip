// Fine stage of VSA: exact softmax attention of each 64-token query cube over
// its K selected 64-token key cubes (64x64 blocks).
//
// bf16 path (the hot loop), one workgroup = 4 waves = one query cube; each
// wave owns 16 query slots (a time slice or an h-row of the cube) and keeps
// their Q fragment in VGPRs; a wave whose slots are all pads computes nothing.
//   * Gather: q, k, v are read either in cube order (64 rows per cube) or
//     straight from raster order, where slot (it, ih, iw) of a cube is row
//     base(cube) + (it*Hh + ih)*Ww + iw, so no reordered copy is needed.
//   * Staging: the 64 K rows and 64 V rows of a key cube go from HBM/L2
//     straight into LDS with buffer_load_dwordx4 ... lds (no VGPRs; the
//     per-lane offsets stay in registers and only a scalar row offset
//     changes from cube to cube, so staging costs no VALU).
//     Each lane's source chunk is chosen so that LDS holds the tiles
//     XOR-swizzled for the reads below; K runs one key cube ahead of V in a
//     2-slot ring each (64 KB at D = 128).  Pad slots of a raster edge cube
//     read their own raster address (a neighbouring token, or zeros past
//     the head's rows): finite values, masked to probability 0.
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: the accumulator then holds,
//     per lane, 16 scores of ONE query row, which is the B-operand layout of
//     O^T += V^T P^T, so probabilities go from the softmax straight into the
//     PV MFMAs.  The V^T operand comes from row-major V by gfx950 transposed
//     LDS reads (ds_read_b64_tr_b16).
//   * Pad key slots: one accumulator init (0 / -inf) masks the (ih, iw) part
//     for every key tile; tiles past the cube's t extent get a -inf offset in
//     the exp2 argument.  Extents come from a per-lane table, one v_readlane
//     per step, and the masks change only when the extent does.
//   * Software pipeline per wave: while the MFMAs of S(n+1) run, the VALU
//     evaluates exp2 of block n; while PV(n) runs, it scales S(n+1) into exp2
//     units (t = s log2(e)/sqrt(d) - m).  The running max m is raised
//     lazily (only when a row exceeds it by 2^8), so probabilities stay
//     <= 256; the common step checks each lane's own maximum against that
//     bound and needs neither the cross-lane row max nor a rescale.
//   * Row sums come from one extra MFMA per k-step against a ones operand.
//   * The epilogue stages O through LDS and writes whole 16-byte chunks,
//     either in cube order or straight to raster order (fusing the inverse
//     reorder), optionally also broadcasting the coarse row of the cube to
//     every valid token (O_coarse in raster order).
// Workgroups are remapped so each XCD walks one contiguous range of
// (head, query cube) tiles, keeping that head's K/V in its own L2.
#include <type_traits>

#include "vsa_internal.h"

namespace vsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
constexpr float inv_sqrt_d() { return D == 64 ? 0.125f : 0.08838834764831845f; }

__device__ inline bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));  // RNE
}

// LDS geometry of one key cube: K and V tiles, both row major [64][D].
// A row is D/8 16-byte chunks.
//  * K is read 16 B per lane down 16 rows (MFMA A operand): chunk c of row r
//    sits at c ^ ksw(r), which puts the 16 rows on 16 distinct chunk
//    positions (256-byte rows) or spreads row pairs over the bank line
//    (128-byte rows, D = 64).
//  * V is read 8 B per lane by transposed reads, 16 rows x 32 bytes per
//    half-wave: chunk c of row r sits at c ^ vsw(r), which makes those 16
//    reads land on distinct bank positions.
template <int D>
struct FineTile {
  static constexpr int kElems = 64 * D;            // elements of a K or V tile
  static constexpr int kKC = D / 8;                // chunks per row
  static constexpr int kDma = kElems / (256 * 8);  // 16-byte DMA loads per thread per tile
  __device__ static constexpr int ksw(int r) { return kKC == 16 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static constexpr int vsw(int r) { return kKC == 16 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); }
};

// Buffer resource over one head of a [rows][D] bf16 tensor.  Reads beyond
// `bytes` return zeros instead of faulting; a head holds at most
// 4096 cubes x 64 rows x 256 bytes, so byte offsets fit 32 bits.
static_assert(int64_t(kMaxCubes) * kSlots * 128 * 2 < (int64_t(1) << 32), "32-bit head offsets");
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const uint16_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);  // raw 32-bit data format
}

// Issues the DMA loads of one tile: thread t moves physical chunks u*256 + t
// from byte offset row_bytes + off[u] of the head.  The LDS destination of a
// load is wave-uniform (M0); lane l lands at +16*l bytes.  The per-lane
// offsets stay in registers across tiles and only the scalar row offset
// changes.  The loads are written as inline assembly so that the compiler
// does not see LDS writes in flight: it would otherwise wait for every
// outstanding DMA before each transposed LDS read (it cannot tell that those
// read another ring slot).  Every consumer of a slot waits for its DMA
// explicitly (s_waitcnt vmcnt(0) + barrier); M0 serves no other purpose in
// these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 is reserved; it is clobbered on purpose
template <int D>
__device__ __forceinline__ void dma_tile(const __amdgpu_buffer_rsrc_t& rs, uint32_t row_bytes,
                                         const uint32_t* off, uint16_t* slot, int wave) {
  const uint32_t lds = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint16_t*)slot));
#pragma unroll
  for (int u = 0; u < FineTile<D>::kDma; ++u)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds + (u * 256 + wave * 64) * 16), "v"(off[u]), "s"(rs), "s"(row_bytes)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Valid extent of a key cube packed as nt | nh << 3 | nw << 6 (each 1..4);
// a full cube packs to kFullExt.
constexpr int kFullExt = 4 | (4 << 3) | (4 << 6);

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

// Masking of pad key slots.  Lane (li, lg) element r of key tile kb is key
// slot 16kb + 4lg + r, i.e. (it, ih, iw) = (kb, lg, r).  The (ih, iw) part
// is the same for every kb: one accumulator init (0 valid, -inf pad) serves
// the first MFMA of every key tile.  The it part masks whole key tiles: it
// enters as a -inf offset of the exp2 argument of tiles kb >= nt.
__device__ __forceinline__ f32x4 hw_bias(int ext, int lg) {
  const int nh = (ext >> 3) & 7, nw = ext >> 6;
  const float vl = lg < nh ? 0.f : -INFINITY;
  return f32x4{vl, nw > 1 ? vl : -INFINITY, nw > 2 ? vl : -INFINITY, nw > 3 ? vl : -INFINITY};
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

// Max over one lane's 16 values (3-input maxes).  The inputs come out of VALU
// arithmetic, so the compiler needs no canonicalising maxes on them.
__device__ __forceinline__ float lane_max(const f32x4* t) {
  const float x = max3f(max3f(t[0][0], t[0][1], t[0][2]), max3f(t[0][3], t[1][0], t[1][1]),
                        max3f(t[1][2], t[1][3], t[2][0]));
  return max3f(x, max3f(t[2][1], t[2][2], t[2][3]), max3f(t[3][0], t[3][1], fmaxf(t[3][2], t[3][3])));
}

// Row max: the lane's max, then over the 4 lanes l, l^16, l^32, l^48 that
// hold the same query row (gfx950 cross-row swaps, no LDS).
__device__ __forceinline__ float row_max(const f32x4* t) {
  float x = lane_max(t);
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// S^T tile of one key cube: sacc[kb] for keys 16kb..16kb+15.  k-step outer,
// key tile inner: 4 independent accumulations between dependent MFMAs.
template <int D>
__device__ __forceinline__ void score_tile(const uint16_t* k_lds, const int* kro, const u32x4* qf,
                                           const f32x4 bias, f32x4* sacc) {
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const u32x4 kf = *reinterpret_cast<const u32x4*>(k_lds + kro[ks] + kb * 16 * D);
      sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf), as_bf16x8(qf[ks]),
                                                         ks == 0 ? bias : sacc[kb], 0, 0, 0);
    }
}

// P^T as the B operand of the PV product: k-step s covers keys
// 32s + 16(i/4) + 4lg + (i%4), i = 0..7 (t already in exp2 units).
__device__ __forceinline__ void probabilities(const f32x4* t, u32x4* pf) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(t[2 * s + (i >> 2)][i & 3]);
    pf[s] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                  pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
  }
}

// O^T[d][q] += V^T[d][keys] P^T[keys][q] and the row sums of P (MFMA
// against ones).  The A operand of lane (li, lg) is V[key][16dt + li] for
// the same 8 keys as pf: a transposed read hands 16 lanes a 16 x 4 block
// supplied as 4 rows x 4 runs of 4 dims, lane s supplying row 4lg + s/4,
// dims 16dt + 4(s%4) .. +3; vtr[dt] holds that address for key tile 0.
template <int D>
__device__ __forceinline__ void pv_tile(const uint16_t* v_lds, const int* vtr, const u32x4* pf,
                                        f32x4* oacc, f32x4& lacc) {
  const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};  // bf16 1.0 x 8
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ones), as_bf16x8(pf[s]), lacc, 0, 0, 0);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      // keys 32s + 4lg + j (elements 0..3) and 32s + 16 + 4lg + j (elements 4..7)
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(v_lds + vtr[dt] + (32 * s) * D));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(v_lds + vtr[dt] + (32 * s + 16) * D));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      const u32x4 a = {l2[0], l2[1], h2[0], h2[1]};
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(pf[s]),
                                                         oacc[dt], 0, 0, 0);
    }
  }
}

// RASTER: q, k, v are raster [B,H,N,D] and o, o_coarse are raster;
// otherwise q, k, v and o are cube order [B,H,Np,D].
// HROWS: wave w owns the 16 query slots of the cube's h-row ih = w (slot
// 16 it + 4 w + iw) instead of its time slice it = w (slots 16w..16w+15); a
// wave whose row or slice lies past the cube's extent holds only pad slots
// and computes nothing.  The launcher takes the mapping that idles more
// waves on the grid at hand.
template <int D, bool RASTER, bool HROWS>
__global__ __launch_bounds__(256, 2) void fine_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx,
    uint16_t* __restrict__ o, float* __restrict__ lse, const uint16_t* __restrict__ oc,
    uint16_t* __restrict__ o_coarse, Geo g) {
  using Tl = FineTile<D>;
  constexpr int kKC = Tl::kKC;
  constexpr int kKS = D / 32;              // k-steps of S^T = K Q^T
  constexpr int kDT = D / 16;              // 16-row tiles of O^T
  constexpr int kT = Tl::kElems;
  constexpr int kOutReg = 64 * kKC / 256;  // 16-byte output chunks per thread
  constexpr int kOS = D + 8;               // padded row stride of the O staging tile
  constexpr float kTau = 8.0f;             // lazy rescale threshold (exp2 units)
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * kT];   // K ring (2), V ring (2)
  uint16_t* const kring = smem;
  uint16_t* const vring = smem + 2 * kT;

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

  // DMA byte offsets (from the cube's first row) of this thread's chunks.
  // A pad slot of a raster edge cube reads its own raster address all the
  // same: a token of a neighbouring row or frame, or past the head's rows,
  // where the buffer resource returns zeros.  Either way a finite value
  // whose probability the masks below make exactly 0.
  uint32_t koff[Tl::kDma], voff[Tl::kDma];
#pragma unroll
  for (int u = 0; u < Tl::kDma; ++u) {
    const int P = u * 256 + tid;
    const int r = P / kKC, c = P % kKC;
    int it, ih, iw;
    dma_slot<D>(u, wave, lane, it, ih, iw);
    const uint32_t rowoff = static_cast<uint32_t>(slot_row<RASTER>(g, it, ih, iw) * D) * 2u;
    koff[u] = rowoff + (c ^ Tl::ksw(r)) * 16;
    voff[u] = rowoff + (c ^ Tl::vsw(r)) * 16;
  }
  // stage K or V of a key cube (first row `row`)
  auto stage = [&](const __amdgpu_buffer_rsrc_t& rs, const uint32_t* off, int row,
                   uint16_t* slot) {
    dma_tile<D>(rs, static_cast<uint32_t>(row) * (D * 2), off, slot, wave);
  };

  // Q fragment: B operand of S^T, lane holds Q[slot 16w+li][32ks + 8lg .. +7]
  u32x4 qf[kKS];
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
    for (int ks = 0; ks < kKS; ++ks) qf[ks] = *reinterpret_cast<const u32x4*>(qrow + 32 * ks + 8 * lg);
  }
  // per-lane LDS element offsets of the operand reads (loop invariant)
  int kro[kKS], vtr[kDT];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) kro[ks] = li * D + (((4 * ks + lg) ^ Tl::ksw(li)) * 8);
  {
    const int r = 4 * lg + (li >> 2);        // V row of key tile 0 this lane supplies
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
      vtr[dt] = r * D + (((2 * dt + ((li & 3) >> 1)) ^ Tl::vsw(r)) * 8) + (li & 1) * 4;
  }

  f32x4 oacc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};

  // key cube extents and first rows, 64 steps per lane vector
  int ext_lanes, row_lanes;
  lane_keys<RASTER>(g, sel, 0, K, lane, ext_lanes, row_lanes);
  auto key_ext = [&](int n) { return __builtin_amdgcn_readlane(ext_lanes, n & 63); };
  auto key_row = [&](int n) { return __builtin_amdgcn_readlane(row_lanes, n & 63); };

  // prologue: K(0), V(0), K(1) in flight together; S(0) and its row max
  const int ext0 = key_ext(0);
  stage(krs, koff, key_row(0), kring);
  stage(vrs, voff, key_row(0), vring);
  if (K > 1) stage(krs, koff, key_row(1), kring + kT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // the masks follow the key cube's extent and are rebuilt only when it changes
  int hw_cur = ext0 >> 3, nt_cur = ext0 & 7;
  f32x4 bias = hw_bias(ext0, lg);
  f32x4 tcur[4];
  // S(0) runs on every wave, also on one past the t extent (its Q rows are
  // redirected to real ones), so that the Q loads are consumed on every path
  // before the loop: the compiler then places no wait for them inside it,
  // where its count of outstanding loads would not include the tile DMA
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) asm volatile("" :: "v"(qf[ks]));   // Q has landed, every path
  score_tile<D>(kring, kro, qf, bias, tcur);
  float mb;     // running row max, exp2 units
  float mbk[4]; // exp2 offset of key tile kb: -mb, or -inf for tiles past the cube's t extent
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    tcur[kb] = kb < nt_cur ? tcur[kb] * c2 : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  mb = row_max(tcur);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    tcur[kb] = tcur[kb] - mb;
    mbk[kb] = kb < nt_cur ? -mb : -INFINITY;
  }

  // One step per selected key cube.  The loop is unrolled by two so that the
  // ring slots (P0 = n & 1) are constants and every LDS address is a
  // register plus an immediate offset.
  auto step = [&](auto p0c, int n) {
    constexpr int P0 = decltype(p0c)::value, P1 = P0 ^ 1;
    // K(n+1) and V(n) have landed for every wave; slots of K(n), V(n-1) are free
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int ext = key_ext(n + 1);
    stage(vrs, voff, key_row(n + 1), vring + P1 * kT);
    if (n + 2 < K) {
      if (((n + 2) & 63) == 0) lane_keys<RASTER>(g, sel, n + 2, K, lane, ext_lanes, row_lanes);
      stage(krs, koff, key_row(n + 2), kring + P0 * kT);
    }
    if (!active) return;
    if ((ext >> 3) != hw_cur) {
      hw_cur = ext >> 3;
      bias = hw_bias(ext, lg);
    }
    if ((ext & 7) != nt_cur) {
      nt_cur = ext & 7;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) mbk[kb] = kb < nt_cur ? -mb : -INFINITY;
    }
    // S(n+1) on the matrix cores while exp2 of block n runs on the VALU
    f32x4 tnext[4];
    score_tile<D>(kring + P1 * kT, kro, qf, bias, tnext);
    u32x4 pf[2];
    probabilities(tcur, pf);
    // PV(n) while S(n+1) is scaled into exp2 units
    pv_tile<D>(vring + P0 * kT, vtr, pf, oacc, lacc);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) tnext[kb][r] = fmaf(tnext[kb][r], c2, mbk[kb]);
    // Every value of the wave within 2^tau of the running max (the common
    // case) needs no row max at all: the cross-lane reduction and the rescale
    // run only when some lane exceeds it.  Wave-uniform branch.
    if (__ballot(lane_max(tnext) > kTau) != 0ull) {
      const float mt = row_max(tnext);
      const bool grow = mt > kTau;
      const float delta = grow ? mt : 0.f;
      const float alpha = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) oacc[dt] *= alpha;
      lacc *= alpha;
      mb += delta;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        tnext[kb] = tnext[kb] - delta;
        mbk[kb] = mbk[kb] - delta;
      }
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) tcur[kb] = tnext[kb];
  };
  for (int n = 0; n + 1 < K; n += 2) {
    step(std::integral_constant<int, 0>{}, n);
    if (n + 2 >= K) break;
    step(std::integral_constant<int, 1>{}, n + 1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (active) {
    u32x4 pf[2];
    probabilities(tcur, pf);
    pv_tile<D>(vring + ((K - 1) & 1) * kT, vtr, pf, oacc, lacc);
  }
  __syncthreads();   // every wave is done with the rings: reuse them for O

  // ---- epilogue: l is the same in every accumulator row of lacc; a wave
  // past the t extent writes zeros (pad rows)
  const float l = lacc[0];
  const float inv = active ? 1.f / l : 0.f;
  if (lse != nullptr && lg == 0)
    lse[bh * g.Np + static_cast<int64_t>(qc) * 64 + qslot] =
        active ? (mb + log2f(l)) * kLn2 : 0.f;

  uint16_t* const o_lds = smem;  // [64][kOS]
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) {
    // lane holds O[q = qslot][d = 16dt + 4lg + r], r = 0..3
    const u32x2 w = {pack_bf16x2(oacc[dt][0] * inv, oacc[dt][1] * inv),
                     pack_bf16x2(oacc[dt][2] * inv, oacc[dt][3] * inv)};
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
struct HalfTile {
  static constexpr int kRows = 32;                 // keys per step
  static constexpr int kElems = kRows * D;         // elements of a K or V half tile
  static constexpr int kKC = D / 8;                // 16-byte chunks per row
  static constexpr int kDma = kElems / (256 * 8);  // 16-byte DMA loads per thread per tile
};

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 is reserved; it is clobbered on purpose
// DMA of one half tile by 256 threads (see dma_tile: same form).
template <int D>
__device__ __forceinline__ void dma_half(const __amdgpu_buffer_rsrc_t& rs, uint32_t row_bytes,
                                         const uint32_t* off, uint16_t* slot, int wave) {
  const uint32_t lds = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint16_t*)slot));
#pragma unroll
  for (int u = 0; u < HalfTile<D>::kDma; ++u)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds + (u * 256 + wave * 64) * 16), "v"(off[u]), "s"(rs), "s"(row_bytes)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// S^T of a half tile for both row blocks: sacc[qb][kb], keys 16kb..16kb+15.
template <int D>
__device__ __forceinline__ void score_half(const uint16_t* k_lds, const int* kro,
                                           const u32x4 (*qf)[D / 32], const f32x4 bias,
                                           f32x4 (*sacc)[2]) {
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const u32x4 kf = *reinterpret_cast<const u32x4*>(k_lds + kro[ks] + kb * 16 * D);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        sacc[qb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(kf), as_bf16x8(qf[qb][ks]), ks == 0 ? bias : sacc[qb][kb], 0, 0, 0);
    }
}

// P^T of a half tile as the B operand of its PV product: element i of row
// block qb is key 16(i/4) + 4lg + i%4 (t in exp2 units).
__device__ __forceinline__ void probabilities_half(const f32x4 (*t)[2], u32x4* pf) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(t[qb][i >> 2][i & 3]);
    pf[qb] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                   pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
  }
}

// O^T += V^T P^T over a half tile and the row sums of P, both row blocks;
// each V^T fragment (two transposed reads) feeds both.
template <int D>
__device__ __forceinline__ void pv_half(const uint16_t* v_lds, const int* vtr, const u32x4* pf,
                                        f32x4 (*oacc)[D / 16], f32x4* lacc) {
  const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};  // bf16 1.0 x 8
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
    lacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ones), as_bf16x8(pf[qb]),
                                                       lacc[qb], 0, 0, 0);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(v_lds + vtr[dt]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(v_lds + vtr[dt] + 16 * D));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    const u32x4 a = {l2[0], l2[1], h2[0], h2[1]};
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
      oacc[qb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(pf[qb]),
                                                             oacc[qb][dt], 0, 0, 0);
  }
}

// Max over one row block of a lane (8 values), and over the row (4 lanes).
__device__ __forceinline__ float lane_max8(const f32x4* t) {
  return max3f(max3f(t[0][0], t[0][1], t[0][2]), max3f(t[0][3], t[1][0], t[1][1]),
               fmaxf(t[1][2], t[1][3]));
}
__device__ __forceinline__ float row_max8(const f32x4* t) {
  float x = lane_max8(t);
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

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
  score_half<D>(kring, kro, qf, bias, tcur);
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
    score_half<D>(kring + P1 * kT, kro, qf, bias, tnext);
    u32x4 pf[2];
    probabilities_half(tcur, pf);
    pv_half<D>(vring + P0 * kT, vtr, pf, oacc, lacc);
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
    probabilities_half(tcur, pf);
    pv_half<D>(vring + kT, vtr, pf, oacc, lacc);   // the last step is a second half
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
    // idle query waves over the cube grid: time slices past T in the last
    // cube layer (4 - nt per cube) or h-rows past Hh in the last cube row
    const int64_t t_idle = int64_t(4 * g.Ct - g.T) * g.Ch * g.Cw;
    const int64_t h_idle = int64_t(4 * g.Ch - g.Hh) * g.Ct * g.Cw;
    auto kern = h_idle > t_idle ? fine_fwd_bf16_kernel<D, RASTER, true>
                                : fine_fwd_bf16_kernel<D, RASTER, false>;
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

hipError_t launch_dense(const Geo& g, const void* q, const void* k, const void* v, void* o,
                        float* lse, hipStream_t s) {
  const dim3 grid(g.B * g.H * ((g.C + 1) / 2)), block(256);
  auto qq = static_cast<const uint16_t*>(q), kk = static_cast<const uint16_t*>(k),
       vv = static_cast<const uint16_t*>(v);
  auto oo = static_cast<uint16_t*>(o);
  if (g.D == 128) return launch_kernel(dense_fwd_bf16_kernel<128>, grid, block, 0, s, qq, kk, vv, oo, lse, g);
  return launch_kernel(dense_fwd_bf16_kernel<64>, grid, block, 0, s, qq, kk, vv, oo, lse, g);
}

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
