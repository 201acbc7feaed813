// Tile building blocks shared by the bf16 attention kernels (the sparse fine
// stage and the dense baseline): operand types, the LDS geometry and swizzles
// of K and V tiles, their DMA into LDS, the S^T = K Q^T and O^T += V^T P^T
// MFMA products over half a key cube, pad-key masks and row maxes.
#pragma once

#include "vsa_internal.h"

namespace vsa {

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

// One half of a key cube's K or V tile: 32 rows, time slices 2h and 2h+1.
template <int D>
struct HalfTile {
  static constexpr int kRows = 32;                 // keys per step
  static constexpr int kElems = kRows * D;         // elements of a K or V half tile
  static constexpr int kKC = D / 8;                // 16-byte chunks per row
  static constexpr int kDma = kElems / (256 * 8);  // 16-byte DMA loads per thread per tile
};

// Issues the DMA loads of one half tile: thread t moves physical chunks
// u*256 + t from byte offset row_bytes + off[u] of the head.  The LDS
// destination of a load is wave-uniform (M0); lane l lands at +16*l bytes.
// The per-lane offsets stay in registers across tiles and only the scalar
// row offset changes.  The loads are written as inline assembly so that the
// compiler does not see LDS writes in flight: it would otherwise wait for
// every outstanding DMA before each transposed LDS read (it cannot tell that
// those read another ring slot).  Every consumer of a slot waits for its DMA
// explicitly (s_waitcnt vmcnt(0) + barrier); M0 serves no other purpose in
// these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 is reserved; it is clobbered on purpose
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

// Valid extent of a key cube packed as nt | nh << 3 | nw << 6 (each 1..4);
// a full cube packs to kFullExt.
constexpr int kFullExt = 4 | (4 << 3) | (4 << 6);

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

// Max over one row block of a lane (8 values, 3-input maxes), and over the
// row: then over the 4 lanes l, l^16, l^32, l^48 that hold the same query
// row (gfx950 cross-row swaps, no LDS).  The inputs come out of VALU
// arithmetic, so the compiler needs no canonicalising maxes on them.
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

// S^T of a half tile (32 keys) for NQ 16-row query blocks: sacc[qb][kb],
// keys 16kb..16kb+15 of the half.  k-step outer, key block inner: 2 NQ
// independent accumulations between dependent MFMAs, and each K fragment
// feeds every row block.
template <int D, int NQ>
__device__ __forceinline__ void score_half(const uint16_t* k_lds, const int* kro,
                                           const u32x4 (*qf)[D / 32], const f32x4 bias,
                                           f32x4 (*sacc)[2]) {
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const u32x4 kf = *reinterpret_cast<const u32x4*>(k_lds + kro[ks] + kb * 16 * D);
#pragma unroll
      for (int qb = 0; qb < NQ; ++qb)
        sacc[qb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(kf), as_bf16x8(qf[qb][ks]), ks == 0 ? bias : sacc[qb][kb], 0, 0, 0);
    }
}

// P^T of a half tile as the B operand of its PV product: element i of row
// block qb is key 16(i/4) + 4lg + i%4 (t in exp2 units).
template <int NQ>
__device__ __forceinline__ void probabilities_half(const f32x4 (*t)[2], u32x4* pf) {
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb) {
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(t[qb][i >> 2][i & 3]);
    pf[qb] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                   pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
  }
}

// O^T[d][q] += V^T[d][keys] P^T[keys][q] over a half tile and the row sums
// of P (MFMA against ones), for NQ row blocks; each V^T fragment (two
// transposed reads) feeds every row block.  The A operand of lane (li, lg)
// is V[key][16dt + li] for the same 8 keys as pf: a transposed read hands 16
// lanes a 16 x 4 block supplied as 4 rows x 4 runs of 4 dims, lane s
// supplying row 4lg + s/4, dims 16dt + 4(s%4) .. +3; vtr[dt] holds that
// address for the half's first 16 keys.
template <int D, int NQ>
__device__ __forceinline__ void pv_half(const uint16_t* v_lds, const int* vtr, const u32x4* pf,
                                        f32x4 (*oacc)[D / 16], f32x4* lacc) {
  const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};  // bf16 1.0 x 8
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb)
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
    for (int qb = 0; qb < NQ; ++qb)
      oacc[qb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(pf[qb]),
                                                             oacc[qb][dt], 0, 0, 0);
  }
}

}  // namespace vsa
