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
// probabilities feed the next MFMA straight from registers).  Tiles reach
// LDS by DMA (buffer loads to LDS) in a 2-slot ring, one barrier per step;
// operands contracted over the token index come from the row-major tiles
// through gfx950 transposed LDS reads (ds_read_b64_tr_b16).
#include <type_traits>

#include "vsa_internal.h"
#include "vsa_bwd.h"
#include "block_lists.h"

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
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef short i16x4 __attribute__((ext_vector_type(4)));

// LDS tile of one 64-token block, row major [64][D], filled by DMA.  It is
// read two ways: 16 bytes per lane down 16 rows (MFMA operands contracted
// over the head dim) and by transposed reads, 8 bytes per lane, 4 rows x 32
// bytes per 16 lanes (operands contracted over the tokens).  gfx950's LDS
// has 64 banks of 4 bytes; measured with the bank-conflict counter, a
// 16-byte read is served in four 16-lane phases, lanes {0-3, 12-15, 20-23,
// 24-27}, {4-11, 16-19, 28-31} and the same sets + 32, and an 8-byte read
// (plain or transposed) in two phases of 32 consecutive lanes.  Chunk c of
// row r sits at c ^ sw(r); sw(r) = 2 (r mod 8) (d = 128) or
// 2 ((r / 2) mod 4) (d = 64) puts every phase of both reads on distinct
// banks.
template <int D>
struct BwdTile {
  static constexpr int kElems = 64 * D;
  static constexpr int kKC = D / 8;                // 16-byte chunks per row
  static constexpr int kDma = kElems / (256 * 8);  // DMA loads per thread per tile
  __device__ static constexpr int sw(int r) { return kKC == 16 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); }
};

// Buffer resource over `bytes` bytes from base (one head of a tensor);
// reads beyond it return zeros.  A head holds at most 2048 cubes x 64 rows
// x 256 bytes, so byte offsets fit 32 bits.
static_assert(int64_t(kMaxCubes) * kSlots * 128 * 2 < (int64_t(1) << 32), "32-bit head offsets");
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);  // raw 32-bit data format
}

// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}

// The DMA loads below are written as inline assembly so that the compiler
// does not see LDS writes in flight: it would otherwise wait for every
// outstanding DMA before each transposed LDS read (it cannot tell that those
// read another ring slot).  Every consumer of a slot waits for its DMA
// explicitly (s_waitcnt vmcnt(0) + barrier); M0 (the LDS destination) serves
// no other purpose in these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 is reserved; it is clobbered on purpose

// DMA of one tile whose first row starts at byte row_bytes of the head:
// thread t moves physical chunks u*256 + t (byte offsets from that row in
// off[]); lane l lands at +16*l bytes of the wave-uniform LDS destination.
// The per-lane offsets stay in registers; only the scalar row offset changes.
template <int D>
__device__ __forceinline__ void dma_rows(const __amdgpu_buffer_rsrc_t& rs, uint32_t row_bytes,
                                         const uint32_t* off, uint16_t* slot, int wave) {
  const uint32_t lds = lds_addr(slot);
#pragma unroll
  for (int u = 0; u < BwdTile<D>::kDma; ++u)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds + (u * 256 + wave * 64) * 16), "v"(off[u]), "s"(rs), "s"(row_bytes)
                 : "memory", "m0");
}
// DMA of 64 fp32 per-slot statistics starting at byte `at` of the head (one
// wave): lane l's value lands at +4*l bytes.
__device__ __forceinline__ void dma_stats(const __amdgpu_buffer_rsrc_t& rs, uint32_t at, float* slot,
                                          int lane) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds_addr(slot)), "v"(static_cast<uint32_t>(lane) * 4u), "s"(rs), "s"(at)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(0) (gfx9 encoding: vmcnt 0, expcnt 7, lgkmcnt 15) as a
// builtin, which the compiler's own wait insertion understands: registers
// loaded before it count as complete, so the loop below them carries no wait
// for them (such a wait would also cover the DMA loads in flight, which the
// compiler does not count).
__device__ __forceinline__ void loads_done() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Row read: 8 consecutive dims of tile row r (r & 15 as for its 16-row
// block), starting at logical chunk c.
template <int D>
__device__ __forceinline__ int row_offset(int r, int c) {
  return r * D + ((c ^ BwdTile<D>::sw(r)) * 8);
}
// Transposed read for an operand contracted over tokens: lane (li, lg) gets
// T[tok][16dt + li] for tok = 32s + 4lg + j (elements 0..3) and
// 32s + 16 + 4lg + j (elements 4..7).  Within 16 lanes, lane m of a
// transposed read receives element m % 4 of the 8-byte runs supplied by
// lanes m/4 + 4j, so lane s supplies row 4lg + s/4, dims 16dt + 4(s%4)..+3;
// tro(dt) is that address for s = 0.
template <int D>
__device__ __forceinline__ int tr_offset(int li, int lg, int dt) {
  const int r = 4 * lg + (li >> 2);
  return row_offset<D>(r, 2 * dt + ((li & 3) >> 1)) + (li & 1) * 4;
}
template <int D>
__device__ __forceinline__ u32x4 tok_read(const uint16_t* t, int tro, int s) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(t + tro + (32 * s) * D));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(t + tro + (32 * s + 16) * D));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

// Writes a [64][D] fp32 tile held in MFMA accumulators to raster rows of a
// cube through LDS, adding an fp32 per-cube row `extra` (scaled by inv_n).
// get(row, d) is evaluated by the owning lane; here the caller has already
// written bf16 rows into `stage` ([64][D+8]).
// RASTER: the cube's valid rows go to their raster rows; otherwise all 64
// cube-order rows are written, zeros on pad slots.
template <int D, bool RASTER>
__device__ __forceinline__ void write_cube_rows(const uint16_t* stage, uint16_t* __restrict__ out,
                                                const Geo& g, int64_t bh, int c, int tid) {
  constexpr int kKC = D / 8, kOS = D + 8, kOutReg = 64 * kKC / 256;
  const CubeExt e = cube_extent(g, c);
#pragma unroll
  for (int u = 0; u < kOutReg; ++u) {
    const int ch = tid + 256 * u, row = ch / kKC, cc = ch % kKC;
    const int64_t tok = slot_token(g, e, row);
    if (RASTER) {
      if (tok >= 0)
        *reinterpret_cast<u32x4*>(out + (bh * g.N + tok) * D + 8 * cc) =
            *reinterpret_cast<const u32x4*>(stage + row * kOS + 8 * cc);
    } else {
      const u32x4 val = tok >= 0 ? *reinterpret_cast<const u32x4*>(stage + row * kOS + 8 * cc)
                                 : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(out + (bh * g.Np + static_cast<int64_t>(c) * kSlots + row) * D +
                                8 * cc) = val;
    }
  }
}

// ---------------------------------------------------------------------------
// Preparation: per slot D = rowsum(dO * O) and lse * log2(e) (+inf on pad
// slots); when the coarse branch has a gradient, per cube also the means of
// q, k, v and the sum of dO_coarse (the coarse backward's operands).  The
// gradient kernels gather q, k, v, dO straight from raster rows.
// Eight workgroups per CU: the C x B*H grid fits one round for the shapes
// of the pages.  Each tensor is summed in its own phase (four loads in
// flight per thread) so that the accumulators stay within 64 VGPRs.
// RASTER = false: q, k, v, dO, O are cube order and dO_coarse is one row per
// cube (the gradient of a per-cube O_coarse), taken as the cube's sum as is.
// MEANS = false: the caller holds the means (those of the forward) and q, k,
// v are not read at all.
template <int D, bool COARSE, bool MEANS, bool RASTER>
__global__ __launch_bounds__(256, 8) void bwd_prep_kernel(BwdPrepArgs a, Geo g) {
  constexpr int kCpr = D / 8;                  // 16-byte chunks per row
  constexpr int kRowsPerPass = 256 / kCpr;
  constexpr int kPasses = kSlots / kRowsPerPass;
  const int c = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const CubeExt e = cube_extent(g, c);
  const int tid = threadIdx.x, chunk = tid % kCpr, row0 = tid / kCpr;
  int64_t rrow[kPasses];   // input row of each pass's slot, -1 for a pad slot
#pragma unroll
  for (int u = 0; u < kPasses; ++u) {
    const int slot = row0 + u * kRowsPerPass;
    const int64_t r = slot_token(g, e, slot);
    rrow[u] = r < 0 ? -1 : RASTER ? bh * g.N + r : bh * g.Np + static_cast<int64_t>(c) * kSlots + slot;
  }
  auto load = [&](const uint16_t* x, int u) {
    return rrow[u] >= 0 ? *reinterpret_cast<const u32x4*>(x + rrow[u] * D + chunk * 8)
                        : u32x4{0u, 0u, 0u, 0u};
  };

  {
    u32x4 dv[kPasses], ov[kPasses];
#pragma unroll
    for (int u = 0; u < kPasses; ++u) {
      dv[u] = load(a.dof, u);
      ov[u] = load(a.o, u);
    }
#pragma unroll
    for (int u = 0; u < kPasses; ++u) {
      float dot = 0.f;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        dot = fmaf(bf16_lo(dv[u][h]), bf16_lo(ov[u][h]), dot);
        dot = fmaf(bf16_hi(dv[u][h]), bf16_hi(ov[u][h]), dot);
      }
#pragma unroll
      for (int o = kCpr / 2; o >= 1; o >>= 1) dot += __shfl_xor(dot, o);
      if (chunk == 0) {
        const int64_t crow = bh * g.Np + static_cast<int64_t>(c) * kSlots + row0 + u * kRowsPerPass;
        a.delta[crow] = dot;
        a.lse2[crow] = rrow[u] >= 0 ? a.lse[crow] * kLog2e : INFINITY;
      }
    }
  }
  if constexpr (COARSE && !MEANS && !RASTER) {
    // nothing to sum: dO_coarse is already one row per cube
    if (tid < D) {
      const int64_t m = (bh * g.C + c) * D + tid;
      a.docs[m] = __uint_as_float(static_cast<uint32_t>(a.doc[m]) << 16);
    }
  } else if constexpr (COARSE) {
    // Column sums of the cube per tensor: the rows of one wave meet by lane
    // shuffles (lanes l, l + kCpr, ... hold the same chunk), the four waves
    // in LDS.  Tensors t0 .. 3 of (q, k, v, dO_coarse per token).
    const int lane = tid & 63, wave = tid >> 6;
    constexpr int kT0 = MEANS ? 0 : 3;
    constexpr int kSums = (RASTER ? 4 : 3) - kT0;
    __shared__ float red[4][kSums][D];       // [wave][tensor - t0][dim]
    const uint16_t* const src[4] = {a.q, a.k, a.v, a.doc};
#pragma unroll
    for (int t = 0; t < kSums; ++t) {
      u32x4 val[kPasses];
#pragma unroll
      for (int u = 0; u < kPasses; ++u) val[u] = load(src[kT0 + t], u);
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
      for (int u = 0; u < kPasses; ++u)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          acc[2 * h] += bf16_lo(val[u][h]);
          acc[2 * h + 1] += bf16_hi(val[u][h]);
        }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int o = kCpr; o < 64; o <<= 1) acc[i] += __shfl_xor(acc[i], o);
      }
      if (lane < kCpr) {
#pragma unroll
        for (int i = 0; i < 8; ++i) red[wave][t][chunk * 8 + i] = acc[i];
      }
    }
    __syncthreads();
    if (tid < D) {
      const float inv_n = 1.f / static_cast<float>(e.nt * e.nh * e.nw);
      float sum[kSums];
#pragma unroll
      for (int t = 0; t < kSums; ++t)
        sum[t] = (red[0][t][tid] + red[1][t][tid]) + (red[2][t][tid] + red[3][t][tid]);
      const int64_t m = (bh * g.C + c) * D + tid;
      if constexpr (MEANS) {
        a.qm[m] = sum[0] * inv_n;
        a.km[m] = sum[1] * inv_n;
        a.vm[m] = sum[2] * inv_n;
      }
      if constexpr (RASTER) a.docs[m] = sum[kSums - 1];
      else a.docs[m] = __uint_as_float(static_cast<uint32_t>(a.doc[m]) << 16);
    }
  }
}

// ---------------------------------------------------------------------------
// Standalone launch of the bitmap transpose (one workgroup per head).
__global__ __launch_bounds__(kBitmapThreads) void idx_transpose_bitmap_kernel(
    const int32_t* __restrict__ idx, int32_t* __restrict__ offsets, int32_t* __restrict__ list,
    int32_t* __restrict__ order, Geo g) {
  extern __shared__ uint32_t bmp[];
  idx_transpose_bitmap(idx, offsets, list, order, g, blockIdx.x, bmp);
}

// ---------------------------------------------------------------------------
// Transposed block lists: for each key cube j of head (b, h), the query cubes
// whose selection contains j, in ascending order.  One workgroup per head:
// count, exclusive scan, then rows are placed R at a time (R <= 32): every
// entry sets its row's bit in a per-key mask (atomicOr, order-free), and its
// position is the key's cursor plus the number of earlier rows of the step
// that hold the same key -- deterministic, no ordering by atomics.
// The dK/dV order of the key cubes stays the identity here.
__global__ __launch_bounds__(256) void idx_transpose_kernel(const int32_t* __restrict__ idx,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ list,
                                                            int32_t* __restrict__ order, Geo g) {
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
    order[bh * C + j] = j;
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
// dQ: one workgroup per query cube, 4 waves x 16 query slots (wave w owns
// h-row ih = w or time slice it = w of the cube, as the forward: HROWS).
// Per selected key cube the K and V tiles go from cube order straight into
// a 2-slot LDS ring by DMA; K^T comes from transposed reads of the K tile.
// Pad key slots get P = 0 as in the forward: a -inf accumulator init for the
// (ih, iw) part, a -inf exp2 offset for key tiles past the cube's t extent,
// extents read per step from a per-lane table.
// tile = bh * C + query cube; smem: 4 K/V tiles, [2 slots][K | V].
template <int D, bool RASTER, bool HROWS>
__device__ __forceinline__ void dq_tile(const BwdFineArgs& a, const Geo& g, int tile,
                                        uint16_t* smem) {
  using Tl = BwdTile<D>;
  constexpr int kKS = D / 32, kDT = D / 16, kOS = D + 8, kT = Tl::kElems;

  const int64_t bh = tile / g.C;
  const int qc = tile % g.C;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int K = g.K;
  const int32_t* __restrict__ sel = a.idx + static_cast<int64_t>(tile) * K;
  const float c2 = inv_sqrt_d<D>() * kLog2e;
  // wave w owns the 16 query slots of h-row ih = w of the cube (slot
  // qslot = 16 (li / 4) + 4 w + li % 4) or of time slice it = w (slot
  // 16 w + li); a wave whose row or slice lies past the grid has no valid
  // query and only stages tiles and meets barriers
  const CubeExt eq = cube_extent(g, qc);
  const int qslot = HROWS ? 16 * (li >> 2) + 4 * wave + (li & 3) : 16 * wave + li;
  const bool active = wave < (HROWS ? eq.nh : eq.nt);   // wave-uniform
  const int64_t qrow = bh * g.Np + static_cast<int64_t>(qc) * 64 + qslot;   // cube-order stats
  const int64_t head0 = bh * (RASTER ? g.N : g.Np) * D;   // q, k, v, dO rows of this head

  // DMA byte offsets (from a key cube's first row) of this thread's chunks;
  // a pad slot of a raster edge cube reads its own raster address (a token
  // of a neighbouring row or frame, or zeros past the head's rows), a
  // finite value whose probability is exactly 0
  uint32_t off[Tl::kDma];
#pragma unroll
  for (int u = 0; u < Tl::kDma; ++u) {
    const int P = u * 256 + tid;
    const int r = P / Tl::kKC;
    int it, ih, iw;
    dma_slot<D>(u, wave, lane, it, ih, iw);
    off[u] = static_cast<uint32_t>(slot_row<RASTER>(g, it, ih, iw) * D) * 2u +
             static_cast<uint32_t>(row_offset<D>(r, P % Tl::kKC) - r * D) * 2u;
  }
  const uint32_t head_bytes = static_cast<uint32_t>((RASTER ? g.N : g.Np) * D * 2);
  const __amdgpu_buffer_rsrc_t krs = head_rsrc(a.k + head0, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc(a.v + head0, head_bytes);
  int rro[kKS], tro[kDT];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) rro[ks] = row_offset<D>(li, 4 * ks + lg);
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) tro[dt] = tr_offset<D>(li, lg, dt);

  u32x4 qf[kKS], df[kKS];
  {
    const int it = qslot >> 4, ih = (qslot >> 2) & 3, iw = qslot & 3;
    const bool valid = it < eq.nt && ih < eq.nh && iw < eq.nw;   // pad rows: P = 0 via lse2
    const int64_t row = cube_row<RASTER>(g, eq, qc) + (valid ? slot_row<RASTER>(g, it, ih, iw) : 0);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      qf[ks] = *reinterpret_cast<const u32x4*>(a.q + head0 + row * D + 32 * ks + 8 * lg);
      df[ks] = *reinterpret_cast<const u32x4*>(a.dof + head0 + row * D + 32 * ks + 8 * lg);
    }
  }
  const float lse2 = a.lse2[qrow];
  const float delta = a.delta[qrow];
  // extents (nt | nh << 3 | nw << 6) and first raster rows of the selected
  // key cubes, 64 steps per lane vector
  constexpr int kFull = 4 | (4 << 3) | (4 << 6);
  int ext_lanes, row_lanes;
  auto keys = [&](int first) {
    const int m = first + lane;
    ext_lanes = kFull;
    row_lanes = 0;
    if (m < K) {
      const CubeExt e = cube_extent(g, sel[m]);
      ext_lanes = e.nt | (e.nh << 3) | (e.nw << 6);
      row_lanes = cube_row<RASTER>(g, e, sel[m]);
    }
  };
  keys(0);
  loads_done();
  int ext_cur = -1;
  f32x4 bias = {0.f, 0.f, 0.f, 0.f};   // (ih, iw) mask of S^T, first MFMA of each key tile
  float offk[4];                        // exp2 offset of key tile kb: -lse2, or -inf past nt
  f32x4 dacc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) dacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // stage K and V of step n
  auto stage = [&](int n, uint16_t* slot) {
    const uint32_t row_bytes = static_cast<uint32_t>(__builtin_amdgcn_readlane(row_lanes, n & 63)) * (D * 2);
    dma_rows<D>(krs, row_bytes, off, slot, wave);
    dma_rows<D>(vrs, row_bytes, off, slot + kT, wave);
  };
  stage(0, smem);
  // one step per selected key cube, unrolled by two so that the ring slot
  // (n & 1) is a constant and LDS addresses are registers plus immediates
  auto step = [&](auto slotc, int n) {
    constexpr int SLOT = decltype(slotc)::value;
    // tiles of key cube n have landed for every wave; the other slot is free
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int ext = __builtin_amdgcn_readlane(ext_lanes, n & 63);
    if (n + 1 < K) {
      if (((n + 1) & 63) == 0) keys(n + 1);
      stage(n + 1, smem + (SLOT ^ 1) * 2 * kT);
    }
    if (!active) return;   // staging only
    const uint16_t* k_t = smem + SLOT * 2 * kT;
    const uint16_t* v_t = k_t + kT;
    if (ext != ext_cur) {
      ext_cur = ext;
      const int nt = ext & 7, nh = (ext >> 3) & 7, nw = ext >> 6;
      const float vl = lg < nh ? 0.f : -INFINITY;
      bias = f32x4{vl, nw > 1 ? vl : -INFINITY, nw > 2 ? vl : -INFINITY, nw > 3 ? vl : -INFINITY};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) offk[kb] = kb < nt ? -lse2 : -INFINITY;
    }
    // S^T first, then dP^T: the exp2 of P runs beside the dP^T MFMAs
    f32x4 sacc[4], pacc[4];
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(k_t + rro[ks] + kb * 16 * D);
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(kf), as_bf16x8(qf[ks]), ks == 0 ? bias : sacc[kb], 0, 0, 0);
      }
    float pp[16];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) pp[kb * 4 + r] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], c2, offk[kb]));
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const u32x4 vf = *reinterpret_cast<const u32x4*>(v_t + rro[ks] + kb * 16 * D);
        pacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(vf), as_bf16x8(df[ks]), ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : pacc[kb], 0, 0, 0);
      }
    // dS^T as the B operand: k-step s covers keys 32s + 16(i/4) + 4lg + (i%4);
    // dQ^T[d][q] += K^T[d][keys] dS^T[keys][q], the second half of dS
    // formed beside the MFMAs of the first
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float ds[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kb = 2 * s + (i >> 2), r = i & 3;
        const float p = pp[kb * 4 + r];
        ds[i] = p * (pacc[kb][r] - delta);
      }
      const u32x4 dsf = {pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]),
                         pack_bf16x2(ds[4], ds[5]), pack_bf16x2(ds[6], ds[7])};
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
        dacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(tok_read<D>(k_t, tro[dt], s)),
                                                           as_bf16x8(dsf), dacc[dt], 0, 0, 0);
    }
  };
  for (int n = 0; n < K; n += 2) {
    step(std::integral_constant<int, 0>{}, n);
    if (n + 1 >= K) break;
    step(std::integral_constant<int, 1>{}, n + 1);
  }
  __syncthreads();   // every wave is done with the ring

  // epilogue: dq[q][d] = scale * acc + dQc[qc][d] / n_qc
  uint16_t* const stage_o = smem;   // rows of skipped waves are pad slots, never written out
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
    if (active) *reinterpret_cast<u32x2*>(stage_o + qslot * kOS + 16 * dt + 4 * lg) = w;
  }
  __syncthreads();
  write_cube_rows<D, RASTER>(stage_o, a.dq, g, bh, qc, tid);
}

// ---------------------------------------------------------------------------
// dK/dV: one workgroup per key cube, wave w owns the 16 keys of h-row
// ih = w (HROWS) or of time slice it = w; a wave whose keys are all pads
// only stages tiles and meets barriers.  The workgroup loops
// over the query cubes that selected this key cube.  Per query cube the Q
// and dO tiles and its 64 lse2 / delta values go straight into a 2-slot LDS
// ring by DMA; Q^T and dO^T come from transposed reads.  Pad query slots
// have lse2 = +inf (P = 0) and zero dO rows, so they add nothing.
// tile = bh * C + rank of the key cube in the head's order (descending
// selection counts); smem: [2 slots][Q | dO]; stat: [slot][lse2 | delta][q].
template <int D, bool RASTER, bool HROWS>
__device__ __forceinline__ void dkdv_tile(const BwdFineArgs& a, const Geo& g, int tile,
                                          uint16_t* smem, float (*stat)[2][64]) {
  using Tl = BwdTile<D>;
  constexpr int kKS = D / 32, kDT = D / 16, kOS = D + 8, kT = Tl::kElems;

  const int64_t bh = tile / g.C;
  const int kc = __builtin_amdgcn_readfirstlane(a.order[bh * g.C + tile % g.C]);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const float c2 = inv_sqrt_d<D>() * kLog2e;
  const int64_t head0 = bh * (RASTER ? g.N : g.Np) * D;   // q, k, v, dO rows of this head
  const int64_t stat0 = bh * g.Np;      // cube-order lse2 / delta of this head

  // DMA byte offsets (from a query cube's first row) of this thread's
  // chunks; a pad slot of a raster edge cube reads its own raster address (a
  // finite value, see dq_tile), and its lse2 of +inf makes its P exactly 0
  uint32_t off[Tl::kDma];
#pragma unroll
  for (int u = 0; u < Tl::kDma; ++u) {
    const int P = u * 256 + tid;
    const int r = P / Tl::kKC;
    int it, ih, iw;
    dma_slot<D>(u, wave, lane, it, ih, iw);
    off[u] = static_cast<uint32_t>(slot_row<RASTER>(g, it, ih, iw) * D) * 2u +
             static_cast<uint32_t>(row_offset<D>(r, P % Tl::kKC) - r * D) * 2u;
  }
  const uint32_t head_bytes = static_cast<uint32_t>((RASTER ? g.N : g.Np) * D * 2);
  const __amdgpu_buffer_rsrc_t qrs = head_rsrc(a.q + head0, head_bytes);
  const __amdgpu_buffer_rsrc_t ors = head_rsrc(a.dof + head0, head_bytes);
  const uint32_t stat_bytes = static_cast<uint32_t>(g.Np * 4);
  const __amdgpu_buffer_rsrc_t lrs = head_rsrc(a.lse2 + stat0, stat_bytes);
  const __amdgpu_buffer_rsrc_t drs = head_rsrc(a.delta + stat0, stat_bytes);
  int rro[kKS], tro[kDT];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) rro[ks] = row_offset<D>(li, 4 * ks + lg);
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) tro[dt] = tr_offset<D>(li, lg, dt);

  // the wave's 16 keys: local key j is slot kslot(j)
  auto kslot = [&](int j) { return HROWS ? 16 * (j >> 2) + 4 * wave + (j & 3) : 16 * wave + j; };
  const CubeExt ek = cube_extent(g, kc);
  const bool active = wave < (HROWS ? ek.nh : ek.nt);   // wave-uniform
  // B operands of S = Q K^T and dP = dO V^T: lane holds (key kslot(li), dims 32ks + 8lg ..)
  u32x4 kf[kKS], vf[kKS];
  {
    const int ks_ = kslot(li);
    const int it = ks_ >> 4, ih = (ks_ >> 2) & 3, iw = ks_ & 3;
    const bool valid = it < ek.nt && ih < ek.nh && iw < ek.nw;   // pad key rows are not written
    const int64_t row = cube_row<RASTER>(g, ek, kc) + (valid ? slot_row<RASTER>(g, it, ih, iw) : 0);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      kf[ks] = *reinterpret_cast<const u32x4*>(a.k + head0 + row * D + 32 * ks + 8 * lg);
      vf[ks] = *reinterpret_cast<const u32x4*>(a.v + head0 + row * D + 32 * ks + 8 * lg);
    }
  }
  f32x4 dkacc[kDT], dvacc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) {
    dkacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dvacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  loads_done();
  const int32_t* off_l = a.offsets + bh * (g.C + 1);
  const int beg = off_l[kc], end = off_l[kc + 1];
  const int32_t* lst = a.list + bh * g.C * g.K;
  // first rows and indices of the listed query cubes, 64 steps per lane
  // vector
  int row_lanes = 0, cube_lanes = 0;
  auto cubes = [&](int first) {   // list positions beg + first ...
    const int m = beg + first + lane;
    row_lanes = 0;
    cube_lanes = 0;
    if (m < end) {
      const int c = lst[m];
      row_lanes = cube_row<RASTER>(g, cube_extent(g, c), c);
      cube_lanes = c;
    }
  };
  // stage Q, dO and the statistics of list position beg + i
  auto stage = [&](int i, int slot) {
    const uint32_t row_bytes = static_cast<uint32_t>(__builtin_amdgcn_readlane(row_lanes, i & 63)) * (D * 2);
    uint16_t* const dst = smem + slot * 2 * kT;
    dma_rows<D>(qrs, row_bytes, off, dst, wave);
    dma_rows<D>(ors, row_bytes, off, dst + kT, wave);
    const uint32_t at = static_cast<uint32_t>(__builtin_amdgcn_readlane(cube_lanes, i & 63)) * (64 * 4);
    if (wave == 0) dma_stats(lrs, at, &stat[slot][0][0], lane);
    if (wave == 1) dma_stats(drs, at, &stat[slot][1][0], lane);
  };
  if (beg < end) {
    cubes(0);
    stage(0, 0);
  }
  // one step per listed query cube, unrolled by two so that the ring slot is
  // a constant and LDS addresses are registers plus immediates
  auto step = [&](auto slotc, int i) {
    constexpr int slot = decltype(slotc)::value;
    const int n = beg + i;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (n + 1 < end) {
      if (((i + 1) & 63) == 0) cubes(i + 1);
      stage(i + 1, slot ^ 1);
    }
    if (!active) return;   // staging only
    const uint16_t* q_t = smem + slot * 2 * kT;
    const uint16_t* o_t = q_t + kT;

    // S and dP: lane holds (q = 16qb + 4lg + r, key = 16w + li).  S first:
    // the exp2 of P runs beside the dP MFMAs, dS beside the dV MFMAs.
    f32x4 sacc[4], pacc[4];
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const u32x4 qa = *reinterpret_cast<const u32x4*>(q_t + rro[ks] + qb * 16 * D);
        sacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(qa), as_bf16x8(kf[ks]), ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[qb], 0, 0, 0);
      }
    // P^T and dS^T as A operands: k-step s covers q = 32s + 16(i/4) + 4lg + (i%4)
    u32x4 pf[2], dsf[2];
    float p[16];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const f32x4 l2 = *reinterpret_cast<const f32x4*>(&stat[slot][0][16 * qb + 4 * lg]);
#pragma unroll
      for (int r = 0; r < 4; ++r) p[4 * qb + r] = __builtin_amdgcn_exp2f(fmaf(sacc[qb][r], c2, -l2[r]));
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
      pf[s] = u32x4{pack_bf16x2(p[8 * s + 0], p[8 * s + 1]), pack_bf16x2(p[8 * s + 2], p[8 * s + 3]),
                    pack_bf16x2(p[8 * s + 4], p[8 * s + 5]), pack_bf16x2(p[8 * s + 6], p[8 * s + 7])};
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const u32x4 oa = *reinterpret_cast<const u32x4*>(o_t + rro[ks] + qb * 16 * D);
        pacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(oa), as_bf16x8(vf[ks]), ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : pacc[qb], 0, 0, 0);
      }
    // dV[key][d] += P^T[key][q] dO[q][d]
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
        dvacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(pf[s]), as_bf16x8(tok_read<D>(o_t, tro[dt], s)), dvacc[dt], 0, 0, 0);
    // dK[key][d] += dS^T[key][q] Q[q][d], the second half of dS formed beside
    // the MFMAs of the first
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float ds[8];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int qb = 2 * s + h;
        const f32x4 dl = *reinterpret_cast<const f32x4*>(&stat[slot][1][16 * qb + 4 * lg]);
#pragma unroll
        for (int r = 0; r < 4; ++r) ds[4 * h + r] = p[4 * qb + r] * (pacc[qb][r] - dl[r]);
      }
      dsf[s] = u32x4{pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]),
                     pack_bf16x2(ds[4], ds[5]), pack_bf16x2(ds[6], ds[7])};
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
        dkacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(dsf[s]), as_bf16x8(tok_read<D>(q_t, tro[dt], s)), dkacc[dt], 0, 0, 0);
    }
  };
  for (int i = 0; beg + i < end; i += 2) {
    step(std::integral_constant<int, 0>{}, i);
    if (beg + i + 1 >= end) break;
    step(std::integral_constant<int, 1>{}, i + 1);
  }
  __syncthreads();   // every wave is done with the ring

  // epilogue: lane holds (key kslot(4lg + r), d = 16dt + li); the rows of a
  // skipped wave are pad slots, never written out
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
      const int key = kslot(4 * lg + r);
      const float xk = dkacc[dt][r] * inv_sqrt_d<D>() + addk;
      const float xv = dvacc[dt][r] + addv;
      stage_k[key * kOS + d] = f32_to_bf16_rne(xk);
      stage_v[key * kOS + d] = f32_to_bf16_rne(xv);
    }
  }
  __syncthreads();
  write_cube_rows<D, RASTER>(stage_k, a.dk, g, bh, kc, tid);
  write_cube_rows<D, RASTER>(stage_v, a.dv, g, bh, kc, tid);
}

// dQ and dK/dV in one launch.  Logical tile t of 2 B H C: per head the C
// dK/dV tiles (longest block lists first) and then its C dQ tiles, so that
// dQ tiles take the slots that the short lists of a head leave free while its
// long lists still run, and both kinds of tile of a head share one XCD's L2
// (every head's q, k, v and dO rows are read by both).
template <int D, bool RASTER, bool HROWS>
__global__ __launch_bounds__(256, 2) void fine_bwd_kernel(BwdFineArgs a, Geo g) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * BwdTile<D>::kElems];
  __shared__ __attribute__((aligned(16))) float stat[2][2][64];
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = t / (2 * g.C), r = t - bh * (2 * g.C);
  if (r < g.C)
    dkdv_tile<D, RASTER, HROWS>(a, g, bh * g.C + r, smem, stat);
  else
    dq_tile<D, RASTER, HROWS>(a, g, bh * g.C + (r - g.C), smem);
}

}  // namespace

namespace {
template <int D, bool RASTER>
hipError_t launch_prep_dim(const Geo& g, const BwdPrepArgs& a, hipStream_t s) {
  const dim3 grid(g.C, g.B * g.H), block(256);
  if (a.doc == nullptr)
    return launch_kernel(bwd_prep_kernel<D, false, false, RASTER>, grid, block, 0, s, a, g);
  if (a.qm == nullptr)
    return launch_kernel(bwd_prep_kernel<D, true, false, RASTER>, grid, block, 0, s, a, g);
  return launch_kernel(bwd_prep_kernel<D, true, true, RASTER>, grid, block, 0, s, a, g);
}
template <bool RASTER>
hipError_t launch_prep_layout(const Geo& g, const BwdPrepArgs& a, hipStream_t s) {
  return g.D == 128 ? launch_prep_dim<128, RASTER>(g, a, s) : launch_prep_dim<64, RASTER>(g, a, s);
}
template <bool RASTER>
hipError_t launch_fine_layout(const Geo& g, const BwdFineArgs& a, hipStream_t s) {
  const dim3 grid(2 * g.B * g.H * g.C), block(256);
  if (waves_hold_h_rows(g))
    return g.D == 128 ? launch_kernel(fine_bwd_kernel<128, RASTER, true>, grid, block, 0, s, a, g)
                      : launch_kernel(fine_bwd_kernel<64, RASTER, true>, grid, block, 0, s, a, g);
  return g.D == 128 ? launch_kernel(fine_bwd_kernel<128, RASTER, false>, grid, block, 0, s, a, g)
                    : launch_kernel(fine_bwd_kernel<64, RASTER, false>, grid, block, 0, s, a, g);
}
}  // namespace

hipError_t launch_bwd_prep(const Geo& g, const BwdPrepArgs& a, bool raster, hipStream_t s) {
  return raster ? launch_prep_layout<true>(g, a, s) : launch_prep_layout<false>(g, a, s);
}

hipError_t launch_idx_transpose(const Geo& g, const int32_t* idx, int32_t* offsets,
                                int32_t* list, int32_t* order, hipStream_t s) {
  if (g.C <= kBitmapCubes) {
    return launch_kernel(idx_transpose_bitmap_kernel, dim3(g.B * g.H), dim3(kBitmapThreads),
                         bitmap_words(g.C) * sizeof(uint32_t), s, idx, offsets, list, order, g);
  }
  return launch_kernel(idx_transpose_kernel, dim3(g.B * g.H), dim3(256),
                       2 * static_cast<size_t>(g.C) * sizeof(int32_t), s, idx, offsets, list,
                       order, g);
}

hipError_t launch_bwd_fine(const Geo& g, const BwdFineArgs& a, bool raster, hipStream_t s) {
  return raster ? launch_fine_layout<true>(g, a, s) : launch_fine_layout<false>(g, a, s);
}

}  // namespace vsa
