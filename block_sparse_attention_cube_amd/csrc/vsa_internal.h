// Internal declarations shared by the HIP kernels and the C-ABI layer.
// Not installed; the public interface is include/vsa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

namespace vsa {

constexpr int kCube = 4;     // cube edge along each of (t, y, x)
constexpr int kSlots = 64;   // tokens per cube
// The coarse stage keeps R x C fp32 score rows in LDS: the forward R = 16
// query cubes per workgroup up to 2048 cubes, R = 8 above; the backward two
// such tiles, R = 8 up to 256 cubes, 16 up to 1216, 8 up to 2048, 4 above.
constexpr int kMaxCubes = 4096;
constexpr int kCoarseBwd16Cubes = 1216;
constexpr int kCoarseBwd8Cubes = 2048;
constexpr int kCoarseBwdSmallCubes = 256;   // up to here the backward takes 8 as well
constexpr int kMaxCubesBackward = kMaxCubes;

// Geometry of one problem, passed by value to every kernel.
struct Geo {
  int B, H, T, Hh, Ww, D;
  int Ct, Ch, Cw, C;
  int K;
  int64_t N, Np;
};

// Cube grid position of cube c and its valid extent per axis (1..4).
struct CubeExt {
  int ct, ch, cw;
  int nt, nh, nw;
};

__host__ __device__ inline CubeExt cube_extent(const Geo& g, int c) {
  CubeExt e;
  e.cw = c % g.Cw;
  e.ch = (c / g.Cw) % g.Ch;
  e.ct = c / (g.Cw * g.Ch);
  e.nt = min(kCube, g.T - kCube * e.ct);
  e.nh = min(kCube, g.Hh - kCube * e.ch);
  e.nw = min(kCube, g.Ww - kCube * e.cw);
  return e;
}

// Raster index of slot s (it*16 + ih*4 + iw) of a cube, or -1 for a pad slot.
__host__ __device__ inline int64_t slot_token(const Geo& g, const CubeExt& e, int s) {
  const int it = s >> 4, ih = (s >> 2) & 3, iw = s & 3;
  if (it >= e.nt || ih >= e.nh || iw >= e.nw) return -1;
  const int64_t t = kCube * e.ct + it, y = kCube * e.ch + ih, x = kCube * e.cw + iw;
  return (t * g.Hh + y) * g.Ww + x;
}

// First input row (within its head) of cube c: 64c in cube order, the token
// of slot (0, 0, 0) in raster order.
template <bool RASTER>
__device__ __forceinline__ int cube_row(const Geo& g, const CubeExt& e, int c) {
  return RASTER ? ((kCube * e.ct) * g.Hh + kCube * e.ch) * g.Ww + kCube * e.cw : kSlots * c;
}
// Row offset of slot (it, ih, iw) from its cube's first row.
template <bool RASTER>
__device__ __forceinline__ int slot_row(const Geo& g, int it, int ih, int iw) {
  return RASTER ? (it * g.Hh + ih) * g.Ww + iw : 16 * it + 4 * ih + iw;
}
// Slot (it, ih, iw) of the u-th 16-byte DMA chunk of thread (wave, lane) of
// a 256-thread workgroup staging a [64][D] bf16 tile: chunk
// P = 256u + 64 wave + lane is row P / (D/8) of the tile.
template <int D>
__device__ __forceinline__ void dma_slot(int u, int wave, int lane, int& it, int& ih, int& iw) {
  if (D == 128) {
    it = u; ih = wave; iw = lane >> 4;
  } else {
    it = 2 * u + (wave >> 1); ih = ((wave & 1) << 1) | (lane >> 5); iw = (lane >> 3) & 3;
  }
}

// fp32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// The rows of a query (or key) cube that the attention kernels give their
// four 16-slot waves: h-rows (slots 16 it + 4 w + iw) when they leave more
// waves idle over the cube grid than time slices (slots 16 w + ..) do, so
// that more waves hold only pad slots and skip their work; time slices
// otherwise.  Idle waves: 4 Ct - T time slices per cube column of the last
// cube layer, 4 Ch - Hh h-rows per cube of the last cube row.
inline bool waves_hold_h_rows(const Geo& g) {
  const int64_t t_idle = int64_t(4 * g.Ct - g.T) * g.Ch * g.Cw;
  const int64_t h_idle = int64_t(4 * g.Ch - g.Hh) * g.Ct * g.Cw;
  return h_idle > t_idle;
}

// Workgroups are dealt to the 8 XCDs round-robin (hardware id w runs on XCD
// w % 8).  Remap so that each XCD receives one contiguous range of logical
// tiles: tiles of one head then share that XCD's L2.
__device__ inline int xcd_remap(int w, int n) {
  constexpr int kXcd = 8;
  const int q = n / kXcd, rem = n % kXcd;
  const int x = w % kXcd, j = w / kXcd;
  return (x < rem) ? x * (q + 1) + j : rem * (q + 1) + (x - rem) * q + j;
}

// Launches kernel k and returns the runtime's verdict on this launch alone
// (unlike hipGetLastError, it neither reads nor clears errors of unrelated
// earlier calls on this thread).
template <typename... P, typename... A>
hipError_t launch_kernel(void (*k)(P...), dim3 grid, dim3 block, size_t lds_bytes,
                         hipStream_t s, A... a) {
  static_assert(sizeof...(P) == sizeof...(A), "argument count");
  std::tuple<P...> args(static_cast<P>(a)...);
  return std::apply(
      [&](auto&... e) {
        void* ptrs[] = {static_cast<void*>(&e)...};
        return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, ptrs,
                               lds_bytes, s);
      },
      args);
}

// ---- launchers (each returns the first HIP launch error, or hipSuccess) ----

// mode 0: raster -> cube order (+ optional fp32 means), mode 1: cube -> raster,
// mode 2: cube order -> fp32 means only, mode 3: raster -> fp32 means only.
// Up to 3 tensors per launch.
struct ReorderBatch {
  const void* x[3];
  void* y[3];
  float* mean[3];
  int count;
};
hipError_t launch_reorder(const Geo& g, int dtype, int mode, const ReorderBatch& b,
                          hipStream_t s);

// Coarse stage from fp32 cube means [B,H,C,D]: scores (optional), softmax,
// O_coarse [B,H,C,D] in dtype, and the top-K index list [B,H,C,K].
hipError_t launch_coarse(const Geo& g, int dtype, const float* qm, const float* km,
                         const float* vm, void* oc, int32_t* idx, float* scores,
                         hipStream_t s);

// Fine stage.  raster = false: q, k, v and o are cube order [B,H,Np,D].
// raster = true: o is raster [B,H,N,D] and, if oc != nullptr, o_coarse
// (raster) receives the per-cube coarse row of every valid token; q, k, v
// are raster [B,H,N,D] for bf16 (gathered by cube in the kernel) and cube
// order for fp32.
hipError_t launch_fine(const Geo& g, int dtype, const void* q, const void* k, const void* v,
                       const int32_t* idx, void* o, float* lse, bool raster,
                       const void* oc, void* o_coarse, hipStream_t s);

// Dense attention over every key cube (bf16, cube order in and out), two
// query cubes per workgroup sharing one key stream; lse optional.
hipError_t launch_dense(const Geo& g, const void* q, const void* k, const void* v, void* o,
                        float* lse, hipStream_t s);

// FP8 (E4M3) copies of bf16 raster q, k, v (D = 128): x[i] raster in,
// y[0], y[1] cube order [B,H,Np,D] bytes (q, k), y[2] per-cube transposed
// V tiles [B,H,C,D,64] bytes, exps int32 [3][B*H*C] (per-cube exponents of
// q, k, v), mean[i] optional fp32 per-cube means [B,H,C,D].
struct Fp8Batch {
  const void* x[3];
  void* y[3];
  float* mean[3];
  int32_t* exps;
};
hipError_t launch_quant_fp8(const Geo& g, const Fp8Batch& b, hipStream_t s);

// FP8 fine stage on the copies above (D = 128); o bf16 in cube order, or
// raster (+ O_coarse broadcast from oc when non-null) for raster = true.
hipError_t launch_fine_fp8(const Geo& g, const void* q8, const void* k8, const void* vt8,
                           const int32_t* exps, const int32_t* idx, void* o, float* lse,
                           bool raster, const void* oc, void* o_coarse, hipStream_t s);

}  // namespace vsa
