// Cube reorder: raster token order <-> cube order, and fp32 per-cube means.
//
// One workgroup moves one 64-token cube of one tensor.  A token row is
// d * sizeof(elem) contiguous bytes in both layouts, so the gather/scatter
// moves whole 16-byte chunks: a wave covers 4 (bf16, d=128) to 16 rows with
// fully coalesced loads and stores.  The forward direction can also sum the
// rows it moves (fp32) and write the mean over the cube's valid slots, so the
// coarse stage needs no second pass over q, k, v.  Bandwidth bound: every
// byte is read once and written once.
#include "vsa_internal.h"

namespace vsa {
namespace {

template <typename T>
struct ChunkOps;

template <>
struct ChunkOps<uint16_t> {  // bfloat16 bits
  static constexpr int kElems = 8;
  __device__ static void add(const uint4& v, float* acc) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += __uint_as_float(w[i] << 16);
      acc[2 * i + 1] += __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

template <>
struct ChunkOps<float> {
  static constexpr int kElems = 4;
  __device__ static void add(const uint4& v, float* acc) {
    acc[0] += __uint_as_float(v.x);
    acc[1] += __uint_as_float(v.y);
    acc[2] += __uint_as_float(v.z);
    acc[3] += __uint_as_float(v.w);
  }
};

// MODE 0: raster -> cube (pads written as zero), optional means.
// MODE 1: cube -> raster (pads dropped).
// MODE 2: cube -> means only.
// MODE 3: raster -> means only (the pooling pass of a forward that gathers
//         q, k, v straight from raster rows).
template <typename T, int D, int MODE>
__global__ __launch_bounds__(256) void reorder_kernel(ReorderBatch b, Geo g) {
  using Ops = ChunkOps<T>;
  constexpr int kE = Ops::kElems;
  constexpr int kCpr = D / kE;               // 16-byte chunks per token row
  constexpr int kRowsPerPass = 256 / kCpr;
  constexpr int kPasses = kSlots / kRowsPerPass;
  static_assert(kSlots % kRowsPerPass == 0, "row split");

  const int tensor = blockIdx.z;
  const int c = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const CubeExt e = cube_extent(g, c);
  const int tid = threadIdx.x;
  const int chunk = tid % kCpr, row0 = tid / kCpr;
  const T* __restrict__ x = static_cast<const T*>(b.x[tensor]);
  T* __restrict__ y = static_cast<T*>(b.y[tensor]);
  float* __restrict__ mean = b.mean[tensor];

  float acc[kE];
#pragma unroll
  for (int i = 0; i < kE; ++i) acc[i] = 0.f;

#pragma unroll
  for (int u = 0; u < kPasses; ++u) {
    const int s = row0 + u * kRowsPerPass;
    const int64_t r = slot_token(g, e, s);
    const int64_t crow = bh * g.Np + (int64_t)c * kSlots + s;
    if (MODE == 0 || MODE == 3) {
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (r >= 0) val = *reinterpret_cast<const uint4*>(x + (bh * g.N + r) * D + chunk * kE);
      if (MODE == 0) *reinterpret_cast<uint4*>(y + crow * D + chunk * kE) = val;
      Ops::add(val, acc);
    } else if (MODE == 1) {
      if (r >= 0) {
        const uint4 val = *reinterpret_cast<const uint4*>(x + crow * D + chunk * kE);
        *reinterpret_cast<uint4*>(y + (bh * g.N + r) * D + chunk * kE) = val;
      }
    } else {
      if (r >= 0) {
        const uint4 val = *reinterpret_cast<const uint4*>(x + crow * D + chunk * kE);
        Ops::add(val, acc);
      }
    }
  }

  if (MODE != 1 && mean != nullptr) {  // uniform across the workgroup
    __shared__ float red[kRowsPerPass][D];
#pragma unroll
    for (int i = 0; i < kE; ++i) red[row0][chunk * kE + i] = acc[i];
    __syncthreads();
    if (tid < D) {
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < kRowsPerPass; ++r) sum += red[r][tid];
      const float n = static_cast<float>(e.nt * e.nh * e.nw);
      mean[(bh * g.C + c) * D + tid] = sum / n;
    }
  }
}

template <typename T, int D>
hipError_t launch_typed(const Geo& g, int mode, const ReorderBatch& b, hipStream_t s) {
  const dim3 grid(g.C, g.B * g.H, b.count), block(256);
  switch (mode) {
    case 0: return launch_kernel(reorder_kernel<T, D, 0>, grid, block, 0, s, b, g);
    case 1: return launch_kernel(reorder_kernel<T, D, 1>, grid, block, 0, s, b, g);
    case 2: return launch_kernel(reorder_kernel<T, D, 2>, grid, block, 0, s, b, g);
    default: return launch_kernel(reorder_kernel<T, D, 3>, grid, block, 0, s, b, g);
  }
}

}  // namespace

hipError_t launch_reorder(const Geo& g, int dtype, int mode, const ReorderBatch& b,
                          hipStream_t s) {
  if (dtype == 1) {
    return g.D == 128 ? launch_typed<uint16_t, 128>(g, mode, b, s)
                      : launch_typed<uint16_t, 64>(g, mode, b, s);
  }
  return g.D == 128 ? launch_typed<float, 128>(g, mode, b, s)
                    : launch_typed<float, 64>(g, mode, b, s);
}

}  // namespace vsa
