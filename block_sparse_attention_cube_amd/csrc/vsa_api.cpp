// C ABI of the VSA library: argument validation, workspace layout and the
// launch sequence of every entry point.  No device memory is allocated here;
// nothing is enqueued until every argument has been checked.
#include "../../include/vsa.h"
#include "vsa_internal.h"
#include "vsa_bwd.h"

#include <initializer_list>
#include <mutex>

namespace {

using vsa::Geo;

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

vsa_status check(const vsa_problem* p) {
  if (p == nullptr) return VSA_ERR_NULL;
  if (p->B < 1 || p->H < 1 || p->T < 1 || p->Hh < 1 || p->Ww < 1) return VSA_ERR_SHAPE;
  if (p->cube_t != vsa::kCube || p->cube_h != vsa::kCube || p->cube_w != vsa::kCube)
    return VSA_ERR_UNSUPPORTED;
  if (p->d != 64 && p->d != 128) return VSA_ERR_UNSUPPORTED;
  if (p->dtype != VSA_F32 && p->dtype != VSA_BF16) return VSA_ERR_UNSUPPORTED;
  const int64_t C = int64_t((p->T + 3) / 4) * ((p->Hh + 3) / 4) * ((p->Ww + 3) / 4);
  if (C > vsa::kMaxCubes) return VSA_ERR_UNSUPPORTED;
  if (p->topk < 1 || p->topk > C) return VSA_ERR_SHAPE;
  const int64_t bh = int64_t(p->B) * p->H;
  if (bh > 65535) return VSA_ERR_UNSUPPORTED;                 // grid y extent
  if (bh * C > (int64_t(1) << 29)) return VSA_ERR_UNSUPPORTED; // 1-D grids of 2 B H C
  // B*H*Np*d elements must stay far from int64 overflow
  if (bh * C * 64 * p->d > (int64_t(1) << 58)) return VSA_ERR_UNSUPPORTED;
  // in-cube raster offsets (elements) are 32-bit: 4 frames of the grid
  if (int64_t(4) * p->Hh * p->Ww * p->d >= (int64_t(1) << 31)) return VSA_ERR_UNSUPPORTED;
  return VSA_OK;
}

Geo geometry(const vsa_problem* p) {
  Geo g;
  g.B = p->B; g.H = p->H; g.T = p->T; g.Hh = p->Hh; g.Ww = p->Ww; g.D = p->d;
  g.Ct = (p->T + 3) / 4; g.Ch = (p->Hh + 3) / 4; g.Cw = (p->Ww + 3) / 4;
  g.C = g.Ct * g.Ch * g.Cw;
  g.K = p->topk;
  g.N = int64_t(p->T) * p->Hh * p->Ww;
  g.Np = int64_t(g.C) * vsa::kSlots;
  return g;
}

size_t elem_bytes(const vsa_problem* p) { return p->dtype == VSA_BF16 ? 2 : 4; }

// Sub-buffers of one workspace, each 256-byte aligned.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    void* r = base ? base + off : nullptr;
    off += round_up(bytes);
    return r;
  }
};

struct FwdWs {
  void* qc; void* kc; void* vc;   // fp32 only: cube-order copies
  float* qm; float* km; float* vm;
  void* oc;
};
// bf16: the fine kernel gathers q, k, v from raster rows, so the forward
// keeps only the per-cube means and O_coarse; fp32 also keeps cube-order
// copies of q, k, v.
FwdWs carve_forward(const vsa_problem* p, void* ws, size_t* total) {
  const Geo g = geometry(p);
  const size_t e = elem_bytes(p);
  const size_t cube = size_t(g.B) * g.H * g.Np * g.D * e;
  const size_t mean = size_t(g.B) * g.H * g.C * g.D * sizeof(float);
  Carver c(ws);
  FwdWs w = {};
  if (p->dtype != VSA_BF16) {
    w.qc = c.take(cube); w.kc = c.take(cube); w.vc = c.take(cube);
  }
  w.qm = static_cast<float*>(c.take(mean));
  w.km = static_cast<float*>(c.take(mean));
  w.vm = static_cast<float*>(c.take(mean));
  w.oc = c.take(size_t(g.B) * g.H * g.C * g.D * e);
  if (total) *total = c.off;
  return w;
}

struct BwdWs {
  float* delta; float* lse2;
  float* qm; float* km; float* vm; float* docs;
  float* stats;
  float* dqc; float* dkc; float* dvc;
  int32_t* offsets; int32_t* list; int32_t* order;
};
BwdWs carve_backward(const vsa_problem* p, void* ws, size_t* total) {
  const Geo g = geometry(p);
  const size_t bh = size_t(g.B) * g.H;
  const size_t mean = bh * g.C * g.D * sizeof(float);
  Carver c(ws);
  BwdWs w;
  w.delta = static_cast<float*>(c.take(bh * g.Np * sizeof(float)));
  w.lse2 = static_cast<float*>(c.take(bh * g.Np * sizeof(float)));
  w.qm = static_cast<float*>(c.take(mean));
  w.km = static_cast<float*>(c.take(mean));
  w.vm = static_cast<float*>(c.take(mean));
  w.docs = static_cast<float*>(c.take(mean));
  w.stats = static_cast<float*>(c.take(3 * bh * g.C * sizeof(float)));
  w.dqc = static_cast<float*>(c.take(mean));
  w.dkc = static_cast<float*>(c.take(mean));
  w.dvc = static_cast<float*>(c.take(mean));
  w.offsets = static_cast<int32_t*>(c.take(bh * (g.C + 1) * sizeof(int32_t)));
  w.list = static_cast<int32_t*>(c.take(bh * size_t(g.C) * g.K * sizeof(int32_t)));
  w.order = static_cast<int32_t*>(c.take(bh * size_t(g.C) * sizeof(int32_t)));
  if (total) *total = c.off;
  return w;
}

// The backward keeps two 16 x C fp32 score tiles of the coarse stage in LDS.
vsa_status check_backward(const vsa_problem* p) {
  const vsa_status st = check(p);
  if (st != VSA_OK) return st;
  if (p->dtype != VSA_BF16) return VSA_ERR_UNSUPPORTED;
  if (geometry(p).C > vsa::kMaxCubesBackward) return VSA_ERR_UNSUPPORTED;
  return VSA_OK;
}

struct CoarseWs { float* qm; float* km; float* vm; };
CoarseWs carve_coarse(const vsa_problem* p, void* ws, size_t* total) {
  const Geo g = geometry(p);
  const size_t mean = size_t(g.B) * g.H * g.C * g.D * sizeof(float);
  Carver c(ws);
  CoarseWs w;
  w.qm = static_cast<float*>(c.take(mean));
  w.km = static_cast<float*>(c.take(mean));
  w.vm = static_cast<float*>(c.take(mean));
  if (total) *total = c.off;
  return w;
}

// FP8 path: bf16 inputs with d = 128 only.
vsa_status check_fp8(const vsa_problem* p) {
  const vsa_status st = check(p);
  if (st != VSA_OK) return st;
  if (p->dtype != VSA_BF16 || p->d != 128) return VSA_ERR_UNSUPPORTED;
  return VSA_OK;
}

struct Fp8Ws {
  void* q8; void* k8; void* vt8; int32_t* exps;
  float* qm; float* km; float* vm;
  void* oc;
};
Fp8Ws carve_forward_fp8(const vsa_problem* p, void* ws, size_t* total) {
  const Geo g = geometry(p);
  const size_t bhc = size_t(g.B) * g.H * g.C;
  const size_t codes = bhc * 64 * g.D;   // one byte per element
  const size_t mean = bhc * g.D * sizeof(float);
  Carver c(ws);
  Fp8Ws w;
  w.q8 = c.take(codes); w.k8 = c.take(codes); w.vt8 = c.take(codes);
  w.exps = static_cast<int32_t*>(c.take(3 * bhc * sizeof(int32_t)));
  w.qm = static_cast<float*>(c.take(mean));
  w.km = static_cast<float*>(c.take(mean));
  w.vm = static_cast<float*>(c.take(mean));
  w.oc = c.take(bhc * g.D * 2);
  if (total) *total = c.off;
  return w;
}

bool misaligned(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0; }

vsa_status pointers(std::initializer_list<const void*> required,
                    std::initializer_list<const void*> optional) {
  for (const void* q : required)
    if (q == nullptr) return VSA_ERR_NULL;
  for (const void* q : required)
    if (misaligned(q)) return VSA_ERR_ALIGN;
  for (const void* q : optional)
    if (q != nullptr && misaligned(q)) return VSA_ERR_ALIGN;
  return VSA_OK;
}

vsa_status workspace(const vsa_problem* p, int op, const void* ws, size_t ws_bytes) {
  const size_t need = vsa_workspace_bytes(p, op);
  if (need == 0) return VSA_OK;
  if (ws == nullptr) return VSA_ERR_NULL;
  if (misaligned(ws)) return VSA_ERR_ALIGN;
  if (ws_bytes < need) return VSA_ERR_WORKSPACE;
  return VSA_OK;
}

vsa_status launched(hipError_t e) { return e == hipSuccess ? VSA_OK : VSA_ERR_LAUNCH; }

// ---- scratch of vsa_forward_static (for callers that cannot allocate) ----
// A file-scope device array holds the forward's workspace.  Each GPU the
// library runs on keeps its own copy until the process ends; its device
// address is looked up once per device (the array's name is only a host-side
// stand-in) and every later call on that device reuses it.  Calls on one
// device share the array: calls that overlap in time on one device race.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices] = {};

vsa_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return VSA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return VSA_ERR_LAUNCH;
    scratch_ptr[dev] = ptr;
  }
  *out = scratch_ptr[dev];
  return VSA_OK;
}

vsa_status forward_launch(const vsa_problem* p, const void* q, const void* k, const void* v,
                          void* o_fine, void* o_coarse, int32_t* idx, float* lse, float* means,
                          void* ws, hipStream_t stream);
vsa_status backward_launch(const vsa_problem* p, const void* q, const void* k, const void* v,
                           const void* o_fine, const float* lse, const int32_t* idx,
                           const float* means, const void* do_fine, const void* do_coarse,
                           void* dq, void* dk, void* dv, void* ws, bool raster,
                           hipStream_t stream);

// The three [B,H,C,d] fp32 blocks of a caller's means buffer [3,B,H,C,d]
// (q, k, v), or the workspace's own when the caller passes none.
struct Means { float* q; float* k; float* v; };
Means means_of(const vsa_problem* p, const float* means, float* wq, float* wk, float* wv) {
  if (means == nullptr) return {wq, wk, wv};
  const Geo g = geometry(p);
  const size_t n = size_t(g.B) * g.H * g.C * g.D;
  float* m = const_cast<float*>(means);
  return {m, m + n, m + 2 * n};
}

}  // namespace

extern "C" {

vsa_status vsa_check_problem(const vsa_problem* p) { return check(p); }

size_t vsa_workspace_bytes(const vsa_problem* p, int op) {
  if (check(p) != VSA_OK) return 0;
  size_t total = 0;
  switch (op) {
    case VSA_OP_FORWARD: carve_forward(p, nullptr, &total); return total;
    case VSA_OP_COARSE: carve_coarse(p, nullptr, &total); return total;
    case VSA_OP_FINE: return 0;
    case VSA_OP_FORWARD_FP8:
      if (check_fp8(p) != VSA_OK) return 0;
      carve_forward_fp8(p, nullptr, &total);
      return total;
    case VSA_OP_BACKWARD:
    case VSA_OP_BACKWARD_CUBE:
      if (check_backward(p) != VSA_OK) return 0;
      carve_backward(p, nullptr, &total);
      return total;
    case VSA_OP_FORWARD_CUBE: carve_coarse(p, nullptr, &total); return total;
    default: return 0;
  }
}

const char* vsa_status_string(vsa_status s) {
  switch (s) {
    case VSA_OK: return "VSA_OK";
    case VSA_ERR_NULL: return "VSA_ERR_NULL: a required pointer is NULL";
    case VSA_ERR_SHAPE: return "VSA_ERR_SHAPE: a dimension is < 1 or topk is outside [1, C]";
    case VSA_ERR_UNSUPPORTED:
      return "VSA_ERR_UNSUPPORTED: head dim, cube size, dtype or problem size not supported";
    case VSA_ERR_ALIGN: return "VSA_ERR_ALIGN: a device pointer is not 16-byte aligned";
    case VSA_ERR_WORKSPACE: return "VSA_ERR_WORKSPACE: workspace smaller than required";
    case VSA_ERR_LAUNCH: return "VSA_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
  }
  return "VSA: unknown status";
}

vsa_status vsa_reorder(const vsa_problem* p, const void* x, void* y, int inverse,
                       hipStream_t stream) {
  vsa_status st = check(p);
  if (st != VSA_OK) return st;
  if ((st = pointers({x, y}, {})) != VSA_OK) return st;
  if (inverse != 0 && inverse != 1) return VSA_ERR_UNSUPPORTED;
  const Geo g = geometry(p);
  vsa::ReorderBatch b = {};
  b.x[0] = x;
  b.y[0] = y;
  b.count = 1;
  return launched(vsa::launch_reorder(g, p->dtype, inverse, b, stream));
}

vsa_status vsa_coarse(const vsa_problem* p, const void* qcube, const void* kcube,
                      const void* vcube, void* o_coarse, int32_t* idx, float* scores,
                      void* ws, size_t ws_bytes, hipStream_t stream) {
  vsa_status st = check(p);
  if (st != VSA_OK) return st;
  if ((st = pointers({qcube, kcube, vcube, o_coarse, idx}, {scores})) != VSA_OK) return st;
  if ((st = workspace(p, VSA_OP_COARSE, ws, ws_bytes)) != VSA_OK) return st;
  const Geo g = geometry(p);
  const CoarseWs w = carve_coarse(p, ws, nullptr);
  vsa::ReorderBatch b = {};
  b.x[0] = qcube; b.x[1] = kcube; b.x[2] = vcube;
  b.mean[0] = w.qm; b.mean[1] = w.km; b.mean[2] = w.vm;
  b.count = 3;
  hipError_t e = vsa::launch_reorder(g, p->dtype, 2, b, stream);
  if (e == hipSuccess)
    e = vsa::launch_coarse(g, p->dtype, w.qm, w.km, w.vm, o_coarse, idx, scores, stream);
  return launched(e);
}

vsa_status vsa_fine(const vsa_problem* p, const void* qcube, const void* kcube,
                    const void* vcube, const int32_t* idx, void* o_fine, float* lse,
                    void* ws, size_t ws_bytes, hipStream_t stream) {
  vsa_status st = check(p);
  if (st != VSA_OK) return st;
  if ((st = pointers({qcube, kcube, vcube, idx, o_fine}, {lse})) != VSA_OK) return st;
  if ((st = workspace(p, VSA_OP_FINE, ws, ws_bytes)) != VSA_OK) return st;
  const Geo g = geometry(p);
  return launched(vsa::launch_fine(g, p->dtype, qcube, kcube, vcube, idx, o_fine, lse,
                                   /*raster=*/false, nullptr, nullptr, stream));
}

vsa_status vsa_fine_raster(const vsa_problem* p, const void* q, const void* k, const void* v,
                           const int32_t* idx, void* o_fine, float* lse, const void* oc,
                           void* o_coarse, hipStream_t stream) {
  vsa_status st = check(p);
  if (st != VSA_OK) return st;
  if (p->dtype != VSA_BF16) return VSA_ERR_UNSUPPORTED;
  if ((oc == nullptr) != (o_coarse == nullptr)) return VSA_ERR_NULL;
  if ((st = pointers({q, k, v, idx, o_fine}, {lse, oc, o_coarse})) != VSA_OK) return st;
  return launched(vsa::launch_fine(geometry(p), p->dtype, q, k, v, idx, o_fine, lse,
                                   /*raster=*/true, oc, o_coarse, stream));
}

vsa_status vsa_dense(const vsa_problem* p, const void* qcube, const void* kcube,
                     const void* vcube, void* o, float* lse, hipStream_t stream) {
  vsa_status st = check(p);
  if (st != VSA_OK) return st;
  if (p->dtype != VSA_BF16) return VSA_ERR_UNSUPPORTED;
  if ((st = pointers({qcube, kcube, vcube, o}, {lse})) != VSA_OK) return st;
  return launched(vsa::launch_dense(geometry(p), qcube, kcube, vcube, o, lse, stream));
}

vsa_status vsa_forward(const vsa_problem* p, const void* q, const void* k, const void* v,
                       void* o_fine, void* o_coarse, int32_t* idx, float* lse, float* means,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  vsa_status st = check(p);
  if (st != VSA_OK) return st;
  if ((st = pointers({q, k, v, o_fine, o_coarse, idx}, {lse, means})) != VSA_OK) return st;
  if ((st = workspace(p, VSA_OP_FORWARD, ws, ws_bytes)) != VSA_OK) return st;
  return forward_launch(p, q, k, v, o_fine, o_coarse, idx, lse, means, ws, stream);
}

vsa_status vsa_forward_static(const vsa_problem* p, const void* q, const void* k, const void* v,
                              void* o_fine, void* o_coarse, int32_t* idx, float* lse,
                              float* means, hipStream_t stream) {
  vsa_status st = check(p);
  if (st != VSA_OK) return st;
  if ((st = pointers({q, k, v, o_fine, o_coarse, idx}, {lse, means})) != VSA_OK) return st;
  if (vsa_workspace_bytes(p, VSA_OP_FORWARD) > kScratchBytes) return VSA_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != VSA_OK) return st;
  return forward_launch(p, q, k, v, o_fine, o_coarse, idx, lse, means, ws, stream);
}

vsa_status vsa_backward(const vsa_problem* p, const void* q, const void* k, const void* v,
                        const void* o_fine, const float* lse, const int32_t* idx,
                        const float* means, const void* do_fine, const void* do_coarse,
                        void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  vsa_status st = check(p);
  if (st != VSA_OK) return st;
  if ((st = pointers({q, k, v, o_fine, lse, idx, do_fine, dq, dk, dv}, {means, do_coarse})) !=
      VSA_OK)
    return st;
  if ((st = check_backward(p)) != VSA_OK) return st;
  if ((st = workspace(p, VSA_OP_BACKWARD, ws, ws_bytes)) != VSA_OK) return st;
  return backward_launch(p, q, k, v, o_fine, lse, idx, means, do_fine, do_coarse, dq, dk, dv, ws,
                         /*raster=*/true, stream);
}

vsa_status vsa_forward_cube(const vsa_problem* p, const void* qcube, const void* kcube,
                            const void* vcube, void* o_fine, void* o_coarse, int32_t* idx,
                            float* lse, float* means, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  vsa_status st = check(p);
  if (st != VSA_OK) return st;
  if ((st = pointers({qcube, kcube, vcube, o_fine, o_coarse, idx}, {lse, means})) != VSA_OK)
    return st;
  if ((st = workspace(p, VSA_OP_FORWARD_CUBE, ws, ws_bytes)) != VSA_OK) return st;
  const Geo g = geometry(p);
  const CoarseWs w = carve_coarse(p, ws, nullptr);
  const Means m = means_of(p, means, w.qm, w.km, w.vm);
  vsa::ReorderBatch b = {};
  b.x[0] = qcube; b.x[1] = kcube; b.x[2] = vcube;
  b.mean[0] = m.q; b.mean[1] = m.k; b.mean[2] = m.v;
  b.count = 3;
  hipError_t e = vsa::launch_reorder(g, p->dtype, 2, b, stream);
  if (e == hipSuccess)
    e = vsa::launch_coarse(g, p->dtype, m.q, m.k, m.v, o_coarse, idx, nullptr, stream);
  if (e == hipSuccess)
    e = vsa::launch_fine(g, p->dtype, qcube, kcube, vcube, idx, o_fine, lse, /*raster=*/false,
                         nullptr, nullptr, stream);
  return launched(e);
}

vsa_status vsa_backward_cube(const vsa_problem* p, const void* qcube, const void* kcube,
                             const void* vcube, const void* o_fine, const float* lse,
                             const int32_t* idx, const float* means, const void* do_fine,
                             const void* do_coarse, void* dq, void* dk, void* dv, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  vsa_status st = check(p);
  if (st != VSA_OK) return st;
  if ((st = pointers({qcube, kcube, vcube, o_fine, lse, idx, do_fine, dq, dk, dv},
                     {means, do_coarse})) != VSA_OK)
    return st;
  if ((st = check_backward(p)) != VSA_OK) return st;
  if ((st = workspace(p, VSA_OP_BACKWARD_CUBE, ws, ws_bytes)) != VSA_OK) return st;
  return backward_launch(p, qcube, kcube, vcube, o_fine, lse, idx, means, do_fine, do_coarse, dq,
                         dk, dv, ws, /*raster=*/false, stream);
}

}  // extern "C"

namespace {

// The launch sequence of vsa_forward on a validated problem and a workspace
// of vsa_workspace_bytes(p, VSA_OP_FORWARD) bytes.
vsa_status forward_launch(const vsa_problem* p, const void* q, const void* k, const void* v,
                          void* o_fine, void* o_coarse, int32_t* idx, float* lse, float* means,
                          void* ws, hipStream_t stream) {
  const Geo g = geometry(p);
  const FwdWs w = carve_forward(p, ws, nullptr);
  const Means m = means_of(p, means, w.qm, w.km, w.vm);   // the caller's buffer, if any
  const bool bf16 = p->dtype == VSA_BF16;
  vsa::ReorderBatch b = {};
  b.x[0] = q; b.x[1] = k; b.x[2] = v;
  b.y[0] = w.qc; b.y[1] = w.kc; b.y[2] = w.vc;
  b.mean[0] = m.q; b.mean[1] = m.k; b.mean[2] = m.v;
  b.count = 3;
  // bf16: pool only (the fine kernel gathers from raster); fp32: cube-order copies + means
  hipError_t e = vsa::launch_reorder(g, p->dtype, bf16 ? 3 : 0, b, stream);
  if (e == hipSuccess)
    e = vsa::launch_coarse(g, p->dtype, m.q, m.k, m.v, w.oc, idx, nullptr, stream);
  if (e == hipSuccess)
    e = vsa::launch_fine(g, p->dtype, bf16 ? q : w.qc, bf16 ? k : w.kc, bf16 ? v : w.vc, idx,
                         o_fine, lse, /*raster=*/true, w.oc, o_coarse, stream);
  return launched(e);
}

// The launch sequence of vsa_backward (raster) or vsa_backward_cube on a
// validated problem and workspace.
vsa_status backward_launch(const vsa_problem* p, const void* q, const void* k, const void* v,
                           const void* o_fine, const float* lse, const int32_t* idx,
                           const float* means, const void* do_fine, const void* do_coarse,
                           void* dq, void* dk, void* dv, void* ws, bool raster,
                           hipStream_t stream) {
  const Geo g = geometry(p);
  const BwdWs w = carve_backward(p, ws, nullptr);
  auto b16 = [](const void* x) { return static_cast<const uint16_t*>(x); };
  vsa::BwdPrepArgs pa;
  pa.q = b16(q); pa.k = b16(k); pa.v = b16(v);
  pa.dof = b16(do_fine); pa.o = b16(o_fine); pa.doc = b16(do_coarse);
  pa.lse = lse;
  pa.delta = w.delta;
  pa.lse2 = w.lse2;
  // with the forward's means the preparation pass does not read q, k, v
  const Means m = means_of(p, means, w.qm, w.km, w.vm);
  pa.qm = means ? nullptr : w.qm; pa.km = means ? nullptr : w.km; pa.vm = means ? nullptr : w.vm;
  pa.docs = w.docs;
  hipError_t e = vsa::launch_bwd_prep(g, pa, raster, stream);
  const bool coarse = do_coarse != nullptr;
  // the coarse backward builds the block lists in spare workgroups when it runs
  if (e == hipSuccess && coarse)
    e = vsa::launch_coarse_bwd(g, m.q, m.k, m.v, w.docs, w.stats, w.dqc, w.dkc, w.dvc, idx,
                               w.offsets, w.list, w.order, stream);
  if (e == hipSuccess && !(coarse && vsa::coarse_bwd_builds_lists(g)))
    e = vsa::launch_idx_transpose(g, idx, w.offsets, w.list, w.order, stream);
  if (e == hipSuccess) {
    vsa::BwdFineArgs fa;
    fa.q = b16(q); fa.k = b16(k); fa.v = b16(v); fa.dof = b16(do_fine);
    fa.lse2 = w.lse2; fa.delta = w.delta; fa.idx = idx;
    fa.offsets = w.offsets; fa.list = w.list; fa.order = w.order;
    fa.dqc = coarse ? w.dqc : nullptr;
    fa.dkc = coarse ? w.dkc : nullptr;
    fa.dvc = coarse ? w.dvc : nullptr;
    fa.dq = static_cast<uint16_t*>(dq);
    fa.dk = static_cast<uint16_t*>(dk);
    fa.dv = static_cast<uint16_t*>(dv);
    e = vsa::launch_bwd_fine(g, fa, raster, stream);
  }
  return launched(e);
}

}  // namespace

extern "C" {

vsa_status vsa_quantize_fp8(const vsa_problem* p, const void* q, const void* k, const void* v,
                            void* q8, void* k8, void* vt8, int32_t* exps, hipStream_t stream) {
  vsa_status st = check_fp8(p);
  if (st != VSA_OK) return st;
  if ((st = pointers({q, k, v, q8, k8, vt8, exps}, {})) != VSA_OK) return st;
  vsa::Fp8Batch b = {};
  b.x[0] = q; b.x[1] = k; b.x[2] = v;
  b.y[0] = q8; b.y[1] = k8; b.y[2] = vt8;
  b.exps = exps;
  return launched(vsa::launch_quant_fp8(geometry(p), b, stream));
}

vsa_status vsa_fine_fp8(const vsa_problem* p, const void* q8, const void* k8, const void* vt8,
                        const int32_t* exps, const int32_t* idx, void* o_fine, float* lse,
                        hipStream_t stream) {
  vsa_status st = check_fp8(p);
  if (st != VSA_OK) return st;
  if ((st = pointers({q8, k8, vt8, exps, idx, o_fine}, {lse})) != VSA_OK) return st;
  return launched(vsa::launch_fine_fp8(geometry(p), q8, k8, vt8, exps, idx, o_fine, lse,
                                       /*raster=*/false, nullptr, nullptr, stream));
}

vsa_status vsa_forward_fp8(const vsa_problem* p, const void* q, const void* k, const void* v,
                           void* o_fine, void* o_coarse, int32_t* idx, float* lse, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  vsa_status st = check_fp8(p);
  if (st != VSA_OK) return st;
  if ((st = pointers({q, k, v, o_fine, o_coarse, idx}, {lse})) != VSA_OK) return st;
  if ((st = workspace(p, VSA_OP_FORWARD_FP8, ws, ws_bytes)) != VSA_OK) return st;
  const Geo g = geometry(p);
  const Fp8Ws w = carve_forward_fp8(p, ws, nullptr);
  vsa::Fp8Batch b = {};
  b.x[0] = q; b.x[1] = k; b.x[2] = v;
  b.y[0] = w.q8; b.y[1] = w.k8; b.y[2] = w.vt8;
  b.mean[0] = w.qm; b.mean[1] = w.km; b.mean[2] = w.vm;
  b.exps = w.exps;
  hipError_t e = vsa::launch_quant_fp8(g, b, stream);
  if (e == hipSuccess)
    e = vsa::launch_coarse(g, p->dtype, w.qm, w.km, w.vm, w.oc, idx, nullptr, stream);
  if (e == hipSuccess)
    e = vsa::launch_fine_fp8(g, w.q8, w.k8, w.vt8, w.exps, idx, o_fine, lse, /*raster=*/true,
                             w.oc, o_coarse, stream);
  return launched(e);
}

}  // extern "C"
