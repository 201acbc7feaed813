// FP8 fine stage: exact softmax attention of each 64-token query cube over
// its K selected key cubes, with q, k, v held as E4M3 codes with per-cube
// power-of-two scales (written by quant_fp8.hip).  The format is this
// library's own; the pages only note that sparse and low-bit attention stack
// (TurboDiffusion write-up, section "主要技术").
//
// One workgroup = 4 waves = one query cube, wave w owns the 16 query
// slots of a time slice (or, where that idles more waves, an h-row) of the
// cube, and a wave whose slots are all pads computes nothing.  A step covers TWO selected key cubes (128 keys), the
// contraction length of gfx950's v_mfma_f32_16x16x128_f8f6f4:
//   * S^T = K Q^T: one MFMA per 16 keys (d = 128 in a single instruction).
//     Lane (li, lg) then holds, for query li, keys 16(b%4) + 4lg + j of
//     cube b/4 in block b, j = 0..3.
//   * Scores go to exp2 units with the per-cube factor
//     2^(eq + ek) log2(e) / sqrt(d); the probabilities P = exp2(t - m) are
//     rounded to E4M3 (v_cvt_pk_fp8_f32) straight into the B operand of
//     O^T += V^T P^T: byte 4b + j of lane (li, lg) is the key of score block
//     b, element j.  The V tile is stored transposed with that key order
//     (byte 16g + 4b + j of row d = key 16b + 4g + j), so the A operand of
//     lane (d row, lg) is one 16-byte read per cube.
//   * The V exponent of each cube is applied by the MFMA itself through its
//     E8M0 operand scales.  The instruction splits the 128-long contraction
//     into 4 blocks of 32: block beta is bytes 16(beta / 2) .. +15 of lane
//     groups 2(beta % 2) and 2(beta % 2) + 1, scaled by the scale operand of
//     lane group beta.  With cube 0 in bytes 0..15 and cube 1 in bytes
//     16..31 every block belongs to one cube: lane groups 0-1 pass cube 0's
//     exponent, 2-3 cube 1's.  Row sums come from one unscaled MFMA of P
//     against ones.
//   * The running max is raised lazily, as in the bf16 kernel: P <= 2^8,
//     well inside E4M3's 448.
//   * K and V^T tiles (8 KB per cube) are staged by buffer_load ... lds DMA
//     into two-slot rings of cube pairs (64 KB), K one step ahead of V.
#include <type_traits>

#include "vsa_internal.h"

namespace vsa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;
constexpr int kTile = 64 * kD;        // bytes of one cube's K tile or V^T tile
constexpr int kPair = 2 * kTile;      // one step: two cubes
constexpr int kDma = kTile / (256 * 16);   // 16-byte DMA loads per thread per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;          // lazy rescale threshold (exp2 units)

static_assert(int64_t(kMaxCubes) * kTile < (int64_t(1) << 32), "32-bit head offsets");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc8(const uint8_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  // the first conversion fills bytes 0-1 and keeps bytes 2-3 of its third
  // operand, which the second overwrites: any value serves there (a's bits
  // cost no register initialisation)
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true));
}

__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b, const f32x4& c) {
  // format 0 (E4M3) for both operands, no block scales
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// DMA of one cube tile: thread t moves physical chunks 256u + t from byte
// offset cube_bytes + off[u] of the head into `slot`; lane l of a wave lands
// at +16 l bytes of the wave's M0 base.  Inline assembly so that the compiler
// does not see the LDS writes (it would otherwise wait for every DMA before
// each LDS read); every consumer waits explicitly (vmcnt(0) + barrier).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 is reserved; it is clobbered on purpose
__device__ __forceinline__ void dma_cube(const __amdgpu_buffer_rsrc_t& rs, uint32_t cube_bytes,
                                         const uint32_t* off, uint8_t* slot, int wave) {
  const uint32_t lds = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)slot));
#pragma unroll
  for (int u = 0; u < kDma; ++u)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds + (u * 256 + wave * 64) * 16), "v"(off[u]), "s"(rs), "s"(cube_bytes)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Masking of pad key slots inside a cube: element j of lane group lg in
// score block b is key slot (it, ih, iw) = (b % 4, lg, j).  The (ih, iw)
// part is the accumulator init of the score MFMA (0 valid, -inf pad); the it
// part is a -inf exp2 offset for blocks b % 4 >= nt.
__device__ __forceinline__ f32x4 hw_bias(int ext, int lg) {
  const int nh = (ext >> 3) & 7, nw = ext >> 6;
  const float vl = lg < nh ? 0.f : -INFINITY;
  return f32x4{nw > 0 ? vl : -INFINITY, nw > 1 ? vl : -INFINITY, nw > 2 ? vl : -INFINITY,
               nw > 3 ? vl : -INFINITY};
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

__device__ __forceinline__ float lane_max(const f32x4* t) {
  float x = -INFINITY;
#pragma unroll
  for (int b = 0; b < 8; ++b) x = max3f(x, fmaxf(t[b][0], t[b][1]), fmaxf(t[b][2], t[b][3]));
  return x;
}

// Row max over the 4 lanes l, l^16, l^32, l^48 holding the same query.
__device__ __forceinline__ float row_max(const f32x4* t) {
  float x = lane_max(t);
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Per-step key data, one step per lane, in two tables: cubes and extents
// (tc = c0 | c1 << 16, tx = ext0 | ext1 << 16), and the exponents
// (te = ek0 | ev0 << 8 | ek1 << 16 | ev1 << 24, each + 128).  A missing
// second cube (odd K) repeats the first with extent 0: every key of it is
// masked.  The loads are issued without branches (a lane past the list
// reads entry 0), and the exponents are loaded separately so that the tile
// DMA, which needs only the cube indices, need not wait for them.
__device__ __forceinline__ void lane_cubes(const Geo& g, const int32_t* __restrict__ sel,
                                           int first, int lane, uint32_t& tc, uint32_t& tx) {
  const int m0 = 2 * (first + lane), m1 = m0 + 1;
  const bool r0 = m0 < g.K, r1 = m1 < g.K;
  const int s0 = sel[r0 ? m0 : 0], s1 = sel[r1 ? m1 : 0];
  const int c0 = min(max(s0, 0), g.C - 1);
  const int c1 = r1 ? min(max(s1, 0), g.C - 1) : c0;
  auto ext = [&](int c, bool real) -> uint32_t {
    if (!real) return 0u;
    const CubeExt e = cube_extent(g, c);
    return static_cast<uint32_t>(e.nt | (e.nh << 3) | (e.nw << 6));
  };
  tc = static_cast<uint32_t>(c0) | (static_cast<uint32_t>(c1) << 16);
  tx = ext(c0, r0) | (ext(c1, r1) << 16);
}

__device__ __forceinline__ uint32_t lane_exps(const int32_t* ek, const int32_t* ev, uint32_t tc) {
  const int c0 = static_cast<int>(tc & 0xffffu), c1 = static_cast<int>(tc >> 16);
  return static_cast<uint32_t>(ek[c0] + 128) | (static_cast<uint32_t>(ev[c0] + 128) << 8) |
         (static_cast<uint32_t>(ek[c1] + 128) << 16) | (static_cast<uint32_t>(ev[c1] + 128) << 24);
}

struct StepKeys {
  int ext[2];
  float c2[2];     // score factor 2^(eq + ek) log2(e) / sqrt(d)
  int vscale;      // E8M0 code of 2^ev of the cube whose PV blocks this lane scales
};

__device__ __forceinline__ StepKeys step_keys(uint32_t x, uint32_t e, float cq, int lg) {
  StepKeys s;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    s.ext[h] = static_cast<int>((x >> (16 * h)) & 511u);
    const int ek = static_cast<int>((e >> (16 * h)) & 255u) - 128;
    // the product of two tiny scales may leave the fp32 range: keep it normal
    s.c2[h] = fmaxf(__builtin_ldexpf(cq, ek), 1.17549435e-38f);
  }
  s.vscale = static_cast<int>((e >> (lg < 2 ? 8 : 24)) & 255u) - 128 + 127;
  return s;
}

// S^T blocks of one cube pair: t[b] for keys 16(b%4).. of cube b/4.
// kro[i]: LDS offset of this lane's i-th 16-byte K chunk in block 0.
__device__ __forceinline__ void scores(const uint8_t* k_lds, const int* kro, const i32x8& qf,
                                       const f32x4* bias, f32x4* t) {
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const uint8_t* base = k_lds + (b >> 2) * kTile + (b & 3) * 16 * kD;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + kro[0]);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + kro[1]);
    const i32x8 kf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    t[b] = mfma_fp8(kf, qf, bias[b >> 2]);
  }
}

// P^T as the B operand: byte 4b + j = exp2(t[b][j]) in E4M3.
__device__ __forceinline__ i32x8 probabilities(const f32x4* t) {
  i32x8 pf;
#pragma unroll
  for (int b = 0; b < 8; ++b)
    pf[b] = static_cast<int>(e4m3x4(__builtin_amdgcn_exp2f(t[b][0]), __builtin_amdgcn_exp2f(t[b][1]),
                                    __builtin_amdgcn_exp2f(t[b][2]), __builtin_amdgcn_exp2f(t[b][3])));
  return pf;
}

// O^T[d][q] += 2^ev V^T[d][keys] P^T[keys][q] over the pair (the V
// exponents as MFMA block scales, E8M0 127 = 1 for P), and the row sums of P
// (every row of lacc).
__device__ __forceinline__ void pv(const uint8_t* v_lds, int vro, const i32x8& pf,
                                   const i32x8& ones, int vscale, f32x4* oacc, f32x4& lacc) {
  lacc = mfma_fp8(ones, pf, lacc);
#pragma unroll
  for (int e = 0; e < kD / 16; ++e) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(v_lds + e * 16 * 64 + vro);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(v_lds + kTile + e * 16 * 64 + vro);
    const i32x8 vf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    oacc[e] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vf, pf, oacc[e], 0, 0, 0, vscale,
                                                               0, 127);
  }
}

// RASTER: o (and o_coarse) are raster [B,H,N,D]; otherwise o is cube order.
// HROWS: wave w owns the 16 query slots of the cube's h-row ih = w instead
// of its time slice it = w; a wave whose row or slice lies past the cube's
// extent holds only pad slots and computes nothing (the launcher takes the
// mapping that idles more waves, as for the bf16 kernel).
template <bool RASTER, bool HROWS>
__global__ __launch_bounds__(256, 2) void fine_fwd_fp8_kernel(
    const uint8_t* __restrict__ q8, const uint8_t* __restrict__ k8,
    const uint8_t* __restrict__ vt8, const int32_t* __restrict__ exps,
    const int32_t* __restrict__ idx, uint16_t* __restrict__ o, float* __restrict__ lse,
    const uint16_t* __restrict__ oc, uint16_t* __restrict__ o_coarse, Geo g) {
  constexpr int kKC = kD / 8;               // 16-byte chunks of a bf16 output row
  constexpr int kOutReg = 64 * kKC / 256;
  constexpr int kOS = kD + 8;
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * kPair];   // K ring (2), V ring (2)
  uint8_t* const kring = smem;
  uint8_t* const vring = smem + 2 * kPair;

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bh = tile / g.C;
  const int qc = tile % g.C;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int K = g.K;
  const int ns = (K + 1) >> 1;
  const int32_t* __restrict__ sel = idx + static_cast<int64_t>(tile) * K;
  const int64_t nbhc = static_cast<int64_t>(g.B) * g.H * g.C;
  const int32_t* ek_head = exps + nbhc + bh * g.C;
  const int32_t* ev_head = exps + 2 * nbhc + bh * g.C;
  const float cq = __builtin_ldexpf(0.08838834764831845f * kLog2e, exps[bh * g.C + qc]);
  const int64_t head0 = bh * g.Np * kD;     // byte offset of this head (all three tensors)
  const uint32_t head_bytes = static_cast<uint32_t>(g.Np * kD);
  const __amdgpu_buffer_rsrc_t krs = rsrc8(k8 + head0, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = rsrc8(vt8 + head0, head_bytes);

  // DMA byte offsets inside a cube tile.  K: row r = P / 8 holds logical
  // chunk (P % 8) ^ ksw(r); V^T: row d = P / 4 holds logical chunk
  // (P % 4) ^ vsw(d).  Both swizzles were chosen by measuring the LDS bank
  // conflict counter of the operand reads (16 lanes reading 16 rows, one
  // 16-byte chunk each) on gfx950: they read with no conflict cycles.  Both
  // use only the low 4 row bits, so the per-lane read offsets hold for every
  // 16-row block.
  auto ksw = [](int r) { return (r & 7) ^ ((r >> 3) & 1); };
  auto vsw = [](int d) { return (d >> 1) & 3; };
  uint32_t koff[kDma], voff[kDma];
#pragma unroll
  for (int u = 0; u < kDma; ++u) {
    const int P = u * 256 + tid;
    const int r = P >> 3, d = P >> 2;
    koff[u] = r * kD + (((P & 7) ^ ksw(r)) * 16);
    voff[u] = d * 64 + (((P & 3) ^ vsw(d)) * 16);
  }
  auto stage = [&](const __amdgpu_buffer_rsrc_t& rs, const uint32_t* off, uint32_t cubes,
                   uint8_t* slot) {
    dma_cube(rs, (cubes & 0xffffu) * static_cast<uint32_t>(kTile), off, slot, wave);
    dma_cube(rs, (cubes >> 16) * static_cast<uint32_t>(kTile), off, slot + kTile, wave);
  };

  // wave w holds time slice w (or h-row w) of the query cube: past the
  // cube's extent its 16 slots are all pads and it computes nothing (it
  // still stages its share of the tiles and meets every barrier).  Lane li
  // serves query slot qslot.
  const CubeExt eq = cube_extent(g, qc);
  const bool active = wave < (HROWS ? eq.nh : eq.nt);
  const int qslot = HROWS ? 16 * (li >> 2) + 4 * wave + (li & 3) : 16 * wave + li;
  // Q fragment (B operand of S^T): Q8[qslot][32lg .. 32lg + 31]
  i32x8 qf;
  {
    const uint8_t* qrow = q8 + head0 + (static_cast<int64_t>(qc) * 64 + qslot) * kD + 32 * lg;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(qrow);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(qrow + 16);
    qf = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  // operand read offsets (loop invariant)
  int kro[2];
  kro[0] = li * kD + (((2 * lg) ^ ksw(li)) * 16);
  kro[1] = li * kD + (((2 * lg + 1) ^ ksw(li)) * 16);
  const int vro = li * 64 + ((lg ^ vsw(li)) * 16);
  const int one4 = 0x38383838;   // E4M3 1.0 x 4
  const i32x8 ones = {one4, one4, one4, one4, one4, one4, one4, one4};

  f32x4 oacc[kD / 16];
#pragma unroll
  for (int e = 0; e < kD / 16; ++e) oacc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};

  uint32_t tab_c, tab_x, tab_e;
  lane_cubes(g, sel, 0, lane, tab_c, tab_x);
  auto rl = [](uint32_t t, int n) {
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(t), n & 63));
  };

  // prologue: K(0), V(0), K(1) in flight together.  The staging needs only
  // the cube indices; the exponent loads (which depend on them) are issued
  // after it and complete under the DMA.
  stage(krs, koff, rl(tab_c, 0), kring);
  stage(vrs, voff, rl(tab_c, 0), vring);
  if (ns > 1) stage(krs, koff, rl(tab_c, 1), kring + kPair);
  tab_e = lane_exps(ek_head, ev_head, tab_c);
  const StepKeys s0 = step_keys(rl(tab_x, 0), rl(tab_e, 0), cq, lg);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int ext_cur[2] = {s0.ext[0], s0.ext[1]};
  f32x4 bias[2] = {hw_bias(s0.ext[0], lg), hw_bias(s0.ext[1], lg)};
  f32x4 tcur[8];
  scores(kring, kro, qf, bias, tcur);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int h = b >> 2;
    const float off = (b & 3) < (s0.ext[h] & 7) ? 0.f : -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) tcur[b][j] = fmaf(tcur[b][j], s0.c2[h], off);
  }
  float mb = row_max(tcur);
#pragma unroll
  for (int b = 0; b < 8; ++b) tcur[b] = tcur[b] - mb;
  int vscale = s0.vscale;
  // exp2 offsets of the 8 key blocks of a step: -mb, or -inf for blocks past
  // their cube's t extent; rebuilt only when an extent changes, lowered with
  // the running max
  int nt_cur[2] = {s0.ext[0] & 7, s0.ext[1] & 7};
  float moff[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) moff[b] = (b & 3) < nt_cur[b >> 2] ? -mb : -INFINITY;

  auto step = [&](auto p0c, int n) {
    constexpr int P0 = decltype(p0c)::value, P1 = P0 ^ 1;
    // K(n+1) and V(n) have landed for every wave; slots of K(n), V(n-1) are free
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const StepKeys sn = step_keys(rl(tab_x, n + 1), rl(tab_e, n + 1), cq, lg);
    stage(vrs, voff, rl(tab_c, n + 1), vring + P1 * kPair);
    if (n + 2 < ns) {
      if (((n + 2) & 63) == 0) {
        lane_cubes(g, sel, n + 2, lane, tab_c, tab_x);
        stage(krs, koff, rl(tab_c, n + 2), kring + P0 * kPair);
        tab_e = lane_exps(ek_head, ev_head, tab_c);
      } else {
        stage(krs, koff, rl(tab_c, n + 2), kring + P0 * kPair);
      }
    }
    if (!active) return;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if ((sn.ext[h] >> 3) != (ext_cur[h] >> 3)) {
        ext_cur[h] = sn.ext[h];
        bias[h] = hw_bias(sn.ext[h], lg);
      }
      if ((sn.ext[h] & 7) != nt_cur[h]) {
        nt_cur[h] = sn.ext[h] & 7;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) moff[4 * h + kb] = kb < nt_cur[h] ? -mb : -INFINITY;
      }
    }
    // S(n+1) on the matrix cores while exp2 of step n runs on the VALU
    f32x4 tnext[8];
    scores(kring + P1 * kPair, kro, qf, bias, tnext);
    const i32x8 pf = probabilities(tcur);
    pv(vring + P0 * kPair, vro, pf, ones, vscale, oacc, lacc);
    // S(n+1) into exp2 units (relative to the running max), pads to -inf
#pragma unroll
    for (int b = 0; b < 8; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) tnext[b][j] = fmaf(tnext[b][j], sn.c2[b >> 2], moff[b]);
    if (__ballot(lane_max(tnext) > kTau) != 0ull) {
      const float mt = row_max(tnext);
      const float delta = mt > kTau ? mt : 0.f;
      const float alpha = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
      for (int e = 0; e < kD / 16; ++e) oacc[e] *= alpha;
      lacc *= alpha;
      mb += delta;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        tnext[b] = tnext[b] - delta;
        moff[b] -= delta;
      }
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) tcur[b] = tnext[b];
    vscale = sn.vscale;
  };
  for (int n = 0; n + 1 < ns; n += 2) {
    step(std::integral_constant<int, 0>{}, n);
    if (n + 2 >= ns) break;
    step(std::integral_constant<int, 1>{}, n + 1);
  }
  {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (active) {
      const i32x8 pf = probabilities(tcur);
      if ((ns - 1) & 1) pv(vring + kPair, vro, pf, ones, vscale, oacc, lacc);
      else pv(vring, vro, pf, ones, vscale, oacc, lacc);
    }
  }
  __syncthreads();   // every wave is done with the rings: reuse them for O

  // a wave past the cube's extent writes zeros (pad rows)
  const float l = lacc[0];   // every row of lacc holds the row sum
  const float inv = active ? 1.f / l : 0.f;
  if (lse != nullptr && lg == 0)
    lse[bh * g.Np + static_cast<int64_t>(qc) * 64 + qslot] = active ? (mb + log2f(l)) * kLn2 : 0.f;

  uint16_t* const o_lds = reinterpret_cast<uint16_t*>(smem);  // [64][kOS]
#pragma unroll
  for (int e = 0; e < kD / 16; ++e) {
    // lane holds O[q = qslot][d = 16e + 4lg + j], j = 0..3
    const u32x2 w = {pack_bf16x2(oacc[e][0] * inv, oacc[e][1] * inv),
                     pack_bf16x2(oacc[e][2] * inv, oacc[e][3] * inv)};
    *reinterpret_cast<u32x2*>(o_lds + qslot * kOS + 16 * e + 4 * lg) = w;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kOutReg; ++u) {
    const int ch = tid + 256 * u, row = ch / kKC, c = ch % kKC;
    const u32x4 val = *reinterpret_cast<const u32x4*>(o_lds + row * kOS + 8 * c);
    if (RASTER) {
      const int64_t tok = slot_token(g, eq, row);
      if (tok >= 0) {
        *reinterpret_cast<u32x4*>(o + (bh * g.N + tok) * kD + 8 * c) = val;
        if (oc != nullptr)
          *reinterpret_cast<u32x4*>(o_coarse + (bh * g.N + tok) * kD + 8 * c) =
              *reinterpret_cast<const u32x4*>(oc + (bh * g.C + qc) * kD + 8 * c);
      }
    } else {
      *reinterpret_cast<u32x4*>(o + (bh * g.Np + static_cast<int64_t>(qc) * 64 + row) * kD + 8 * c) = val;
    }
  }
}

}  // namespace

hipError_t launch_fine_fp8(const Geo& g, const void* q8, const void* k8, const void* vt8,
                           const int32_t* exps, const int32_t* idx, void* o, float* lse,
                           bool raster_out, const void* oc, void* o_coarse, hipStream_t s) {
  if (g.D != kD) return hipErrorInvalidValue;
  const dim3 grid(g.B * g.H * g.C), block(256);
  auto u8 = [](const void* p) { return static_cast<const uint8_t*>(p); };
  const bool hrows = waves_hold_h_rows(g);
  auto kern = raster_out ? (hrows ? fine_fwd_fp8_kernel<true, true> : fine_fwd_fp8_kernel<true, false>)
                         : (hrows ? fine_fwd_fp8_kernel<false, true> : fine_fwd_fp8_kernel<false, false>);
  return launch_kernel(kern, grid, block, 0, s, u8(q8), u8(k8), u8(vt8), exps, idx,
                       static_cast<uint16_t*>(o), lse, static_cast<const uint16_t*>(oc),
                       static_cast<uint16_t*>(o_coarse), g);
}

}  // namespace vsa
