// Transposed block lists of one head from a C x C bit matrix in LDS (the
// backward's key-major view of the selection), shared by the standalone
// kernel and the coarse backward, which runs it in spare workgroups.
#pragma once
#include "vsa_internal.h"
#include "vsa_bwd.h"

namespace vsa {

// Transposed block lists for C <= kBitmapCubes: the whole selection of a head
// becomes a C x C bit matrix in LDS, row j holding the query cubes that
// selected key cube j.  Counts are row popcounts, and every entry (i, j)
// finds its position directly: offset of j plus the number of set bits below
// bit i of row j.  A few barriers instead of one round per few rows.
// Run by a 1024-thread workgroup for head bh, with bitmap_words(C) words of
// LDS at bmp.
constexpr int kBitmapThreads = 1024;
__host__ __device__ inline size_t bitmap_words(int C) {
  return static_cast<size_t>(C) * ((C + 31) / 32) + 2 * static_cast<size_t>(C);
}
__device__ inline void idx_transpose_bitmap(const int32_t* __restrict__ idx,
                                            int32_t* __restrict__ offsets,
                                            int32_t* __restrict__ list, int32_t* __restrict__ order,
                                            const Geo& g, int64_t bh, uint32_t* bmp) {
  constexpr int kNT = kBitmapThreads, kBatch = 4;
  const int C = g.C, K = g.K, W = (C + 31) / 32;
  uint32_t* bits = bmp;                                        // [C][W]
  int32_t* start = reinterpret_cast<int32_t*>(bmp + C * W);    // [C]: counts, then offsets
  int32_t* cnt = start + C;                                     // [C]: counts
  const int tid = threadIdx.x;
  const int n = C * K;
  const int32_t* rows = idx + bh * n;
  for (int e = tid; e < C * W; e += kNT) bits[e] = 0u;
  __syncthreads();
  // entries in batches: the loads of a batch are in flight together
  for (int e0 = tid; e0 < n; e0 += kBatch * kNT) {
    int j[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) j[u] = e0 + u * kNT < n ? rows[e0 + u * kNT] : -1;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = (e0 + u * kNT) / K;
      if (j[u] >= 0) atomicOr(&bits[j[u] * W + (i >> 5)], 1u << (i & 31));   // entries of a row are distinct
    }
  }
  __syncthreads();
  for (int jj = tid; jj < C; jj += kNT) {
    int c = 0;
    for (int w = 0; w < W; ++w) c += __popc(bits[jj * W + w]);
    start[jj] = c;
    cnt[jj] = c;
  }
  __syncthreads();
  // exclusive scan of the C <= 512 counts on wave 0: 8 per lane, then the lanes
  if (tid < 64) {
    int v[8], run = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int jj = tid * 8 + u;
      v[u] = jj < C ? start[jj] : 0;
      run += v[u];
    }
    int incl = run;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (tid >= d) incl += y;
    }
    int ex = incl - run;
    int32_t* off = offsets + bh * (C + 1);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int jj = tid * 8 + u;
      if (jj < C) {
        start[jj] = ex;
        off[jj] = ex;
      }
      ex += v[u];
    }
    if (tid == 0) off[C] = n;
  }
  __syncthreads();
  // key cubes by descending count, ties by index (heaviest dK/dV work first)
  for (int jj = tid; jj < C; jj += kNT) {
    const int cj = cnt[jj];
    int rank = 0;
    for (int t = 0; t < C; ++t) {
      const int ct = cnt[t];
      rank += (ct > cj) | ((ct == cj) & (t < jj));
    }
    order[bh * C + rank] = jj;
  }
  int32_t* out = list + bh * n;
  for (int e0 = tid; e0 < n; e0 += kBatch * kNT) {
    int j[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) j[u] = e0 + u * kNT < n ? rows[e0 + u * kNT] : -1;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (j[u] < 0) continue;
      const int i = (e0 + u * kNT) / K;
      const uint32_t* row = bits + j[u] * W;
      int rank = __popc(row[i >> 5] & ((1u << (i & 31)) - 1u));
      for (int w = 0; w < (i >> 5); ++w) rank += __popc(row[w]);
      out[start[j[u]] + rank] = i;
    }
  }
}


}  // namespace vsa
