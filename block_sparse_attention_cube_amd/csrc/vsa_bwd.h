// Internal declarations of the backward kernels (not installed).
#pragma once

#include "vsa_internal.h"

namespace vsa {

// Preparation pass (bf16): raster tensors, or cube-order tensors with a
// per-cube dO_coarse [B,H,C,D] (raster = false).
struct BwdPrepArgs {
  const uint16_t* q; const uint16_t* k; const uint16_t* v;
  const uint16_t* dof;   // upstream gradient of O_fine
  const uint16_t* o;     // O_fine
  const uint16_t* doc;   // upstream gradient of O_coarse, or nullptr (zero)
  const float* lse;      // [B,H,Np] forward log-sum-exp (natural log)
  float* delta;          // [B,H,Np] rowsum(dO * O), 0 on pad slots
  float* lse2;           // [B,H,Np] lse * log2(e), +inf on pad slots (their P is 0)
  float* qm; float* km; float* vm;   // [B,H,C,D] means over valid slots, or all
                                     // nullptr when the caller holds them
  float* docs;           // [B,H,C,D] sums of dO_coarse over valid slots
};
hipError_t launch_bwd_prep(const Geo& g, const BwdPrepArgs& a, bool raster, hipStream_t s);

// Coarse-stage gradients from the means (fp32): dqc/dkc/dvc [B,H,C,D] and row
// statistics stats [3][B,H,C] (row max, row sum of exp, rowsum(P * dP)).
// With idx set and C <= 512 it also builds the transposed block lists (as
// launch_idx_transpose) in spare workgroups of its first kernel.
hipError_t launch_coarse_bwd(const Geo& g, const float* qm, const float* km, const float* vm,
                             const float* docs, float* stats, float* dqc, float* dkc,
                             float* dvc, const int32_t* idx, int32_t* offsets, int32_t* list,
                             int32_t* order, hipStream_t s);
// Cube counts up to which the block lists come from a bit matrix in LDS (one
// 1024-thread workgroup per head); launch_coarse_bwd builds them then.
constexpr int kBitmapCubes = 512;
inline bool coarse_bwd_builds_lists(const Geo& g) { return g.C <= kBitmapCubes; }

// offsets [B,H,C+1], list [B,H,C*K]: query cubes selecting each key cube;
// order [B,H,C]: the key cubes of each head by descending selection count
// (ties by index), the order the dK/dV workgroups take them in.
hipError_t launch_idx_transpose(const Geo& g, const int32_t* idx, int32_t* offsets,
                                int32_t* list, int32_t* order, hipStream_t s);

struct BwdFineArgs {
  const uint16_t* q; const uint16_t* k; const uint16_t* v; const uint16_t* dof;   // rows
  const float* lse2;     // [B,H,Np] lse * log2(e), +inf on pad slots
  const float* delta;    // [B,H,Np]
  const int32_t* idx;    // [B,H,C,K]
  const int32_t* offsets; const int32_t* list; const int32_t* order;
  const float* dqc; const float* dkc; const float* dvc;   // coarse gradients or nullptr
  uint16_t* dq; uint16_t* dk; uint16_t* dv;               // out, layout of the inputs
};
// raster = false: q, k, v, dO in cube order [B,H,Np,D], dq/dk/dv written in
// cube order with zero pad rows.
hipError_t launch_bwd_fine(const Geo& g, const BwdFineArgs& a, bool raster, hipStream_t s);

}  // namespace vsa
