/*
 * vsa.h -- C ABI of the MI355X (gfx950) video sparse attention library.
 *
 * Video sparse attention (VSA) is a trainable, dynamic block-sparse attention
 * that drops in for FlashAttention inside a video diffusion transformer
 * (FastWan/VSA re-post on yumynutrition.com, section
 * "传统零散郑重力，为何会在蒸馏中失效？").  A coarse stage decides a
 * block-sparse pattern of 64x64 blocks and a fine block-sparse kernel runs
 * exact attention over it (same page, results section "一张卡，秒生视频": the
 * fine-kernel, coarse-overhead and 64x64 FlexAttention lines, Fig. 5).
 *
 * Geometry.  q/k/v come in raster token order [B, H, N, d] with
 * N = T*Hh*Ww and token r = (t*Hh + y)*Ww + x.  A 64-token block is a 4x4x4
 * cube.  Each axis is padded at its high end to a multiple of 4, giving a
 * cube grid (Ct, Ch, Cw) = (ceil(T/4), ceil(Hh/4), ceil(Ww/4)), C = Ct*Ch*Cw
 * cubes and Np = 64*C padded tokens.  In "cube order" position
 * p = 64*c + it*16 + ih*4 + iw, with c = (ct*Ch + ch)*Cw + cw, holds token
 * (4ct+it, 4ch+ih, 4cw+iw); a position outside the real grid is a pad slot.
 * Pad slots are zero in reorder outputs and are never attended to.
 *
 * Method (each stage restated in the entry point that runs it):
 *   coarse:  Qc, Kc, Vc = mean over the valid slots of each cube (fp32);
 *            Sc = Qc Kc^T / sqrt(d); O_coarse per cube = softmax_row(Sc) Vc;
 *            idx[i] = the K key cubes with the largest Sc[i, :], ties to the
 *            lower cube index, listed in ascending cube order.
 *   fine:    for every query slot of cube i, exact softmax attention with
 *            scale 1/sqrt(d) over the valid key slots of the cubes idx[i].
 * Sparsity is 1 - K/C (8x fewer attention FLOPs at 87.5%, results section,
 * 410M scaling experiment).
 *
 * Conventions shared by every entry point.
 *   - All tensors are contiguous, d innermost, in the problem's dtype unless
 *     stated: VSA_BF16 (bfloat16) or VSA_F32.  idx is int32, lse is fp32
 *     natural-log log-sum-exp.
 *   - The caller owns every buffer.  The library never allocates or frees
 *     device memory, keeps no pointer after returning and holds no mutable
 *     global state (vsa_forward_static's device array aside); calls are
 *     re-entrant.  Device pointers must point to memory of the current HIP
 *     device.
 *   - Inputs (q, k, v, o_fine and the upstream gradients) must be finite.  A
 *     pad slot of an edge cube is staged from its own raster address, which
 *     holds a token of a neighbouring row or frame (or reads as zero past the
 *     head's rows); its probability is exactly 0, so a finite value there
 *     changes nothing, but a NaN or Inf would spread.
 *   - All work is enqueued asynchronously on `stream` (0 = null stream); the
 *     library never synchronises with the host.  Buffers must stay alive
 *     until the stream has executed the work.
 *   - Every argument is validated before anything is enqueued.  On any error
 *     nothing is enqueued and outputs are untouched.  Device pointers must be
 *     16-byte aligned (VSA_ERR_ALIGN).  Limits: B, H, T, Hh, Ww >= 1;
 *     cube = 4x4x4 (else VSA_ERR_UNSUPPORTED); d in {64, 128}
 *     (else VSA_ERR_UNSUPPORTED); 1 <= topk <= C (else VSA_ERR_SHAPE);
 *     C <= 4096 cubes, B*H <= 65535, B*H*C <= 2^29, B*H*Np*d < 2^58 and
 *     4*Hh*Ww*d < 2^31 (else VSA_ERR_UNSUPPORTED).
 *   - A kernel launch failure is reported as VSA_ERR_LAUNCH.
 *   - Offsets are 64-bit throughout.
 */
#ifndef VSA_H_
#define VSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VSA_OK = 0,
  VSA_ERR_NULL = 1,         /* a required pointer is NULL                       */
  VSA_ERR_SHAPE = 2,        /* a dimension is < 1 or topk is outside [1, C]      */
  VSA_ERR_UNSUPPORTED = 3,  /* valid but not implemented: d, cube size, dtype    */
  VSA_ERR_ALIGN = 4,        /* a device pointer is not 16-byte aligned           */
  VSA_ERR_WORKSPACE = 5,    /* workspace smaller than vsa_workspace_bytes()      */
  VSA_ERR_LAUNCH = 6        /* the HIP runtime rejected a kernel launch          */
} vsa_status;

typedef enum { VSA_F32 = 0, VSA_BF16 = 1 } vsa_dtype;

typedef struct {
  int32_t B, H;              /* batch, heads                                     */
  int32_t T, Hh, Ww;         /* token grid; N = T*Hh*Ww                          */
  int32_t d;                 /* head dimension: 64 or 128                        */
  int32_t cube_t, cube_h, cube_w;  /* cube edge per axis; must be 4, 4, 4      */
  int32_t topk;              /* key cubes kept per query cube, 1 <= topk <= C    */
  int32_t dtype;             /* vsa_dtype of q, k, v and of every output tensor  */
} vsa_problem;

enum { VSA_OP_FORWARD = 0, VSA_OP_BACKWARD = 1, VSA_OP_COARSE = 2, VSA_OP_FINE = 3,
       VSA_OP_FORWARD_FP8 = 4, VSA_OP_FORWARD_CUBE = 5, VSA_OP_BACKWARD_CUBE = 6 };

/* Bytes of device workspace the entry point `op` needs for problem `p`
 * (VSA_OP_FORWARD: vsa_forward, VSA_OP_BACKWARD: vsa_backward,
 * VSA_OP_COARSE: vsa_coarse, VSA_OP_FINE: vsa_fine,
 * VSA_OP_FORWARD_FP8: vsa_forward_fp8, VSA_OP_FORWARD_CUBE: vsa_forward_cube,
 * VSA_OP_BACKWARD_CUBE: vsa_backward_cube).  Returns 0 if `p` is
 * invalid (see vsa_check_problem) or `op` unknown; a valid problem may also
 * need 0 bytes (then ws may be NULL).  Host-only, never touches the GPU. */
size_t vsa_workspace_bytes(const vsa_problem* p, int op);

/* Validates `p` alone (host-only).  Returns the status every entry point
 * would return for this problem with valid pointers. */
vsa_status vsa_check_problem(const vsa_problem* p);

/* Cube reorder (the 64-token blocks of the results section, laid out as 4x4x4
 * cubes).
 *   inverse = 0: x raster [B,H,N,d] -> y cube order [B,H,Np,d]; pad slots of
 *                y are written as zero.
 *   inverse = 1: x cube order [B,H,Np,d] -> y raster [B,H,N,d]; pad slots of
 *                x are ignored.
 * A pure permutation: bit-exact.  x and y must not overlap.  Any other
 * inverse value returns VSA_ERR_UNSUPPORTED. */
vsa_status vsa_reorder(const vsa_problem* p, const void* x, void* y, int inverse,
                       hipStream_t stream);

/* Coarse stage on cube-order inputs (block pattern producer of the results
 * section, Fig. 5).
 *   qcube, kcube, vcube : [B,H,Np,d] cube order, pad slots ignored.
 *   o_coarse            : [B,H,C,d] out, softmax_row(Sc) Vc per query cube.
 *   idx                 : [B,H,C,topk] int32 out, ascending cube indices.
 *   scores              : [B,H,C,C] fp32 out (Sc), or NULL to skip.
 *   ws, ws_bytes        : workspace of vsa_workspace_bytes(p, VSA_OP_COARSE).
 * Means, scores, softmax and O_coarse are computed in fp32; the selection
 * compares fp32 scores exactly (-0 equals +0). */
vsa_status vsa_coarse(const vsa_problem* p, const void* qcube, const void* kcube,
                      const void* vcube, void* o_coarse, int32_t* idx, float* scores,
                      void* ws, size_t ws_bytes, hipStream_t stream);

/* Fine stage on cube-order inputs (the fine block-sparse kernel of the
 * results section).
 *   qcube, kcube, vcube : [B,H,Np,d] cube order; pad slots of kcube/vcube are
 *                         never attended to but must hold finite values
 *                         (vsa_reorder writes zeros there).
 *   idx                 : [B,H,C,topk] int32, each in [0, C), distinct per row
 *                         (any order; the result does not depend on it).
 *   o_fine              : [B,H,Np,d] out, cube order.  Rows of pad slots are
 *                         written with unspecified values.
 *   lse                 : [B,H,Np] fp32 out (natural log), or NULL.
 *   ws, ws_bytes        : workspace of vsa_workspace_bytes(p, VSA_OP_FINE)
 *                         (currently 0 bytes; ws may then be NULL).
 * bf16 inputs use bf16 MFMA with fp32 accumulation and fp32 softmax; fp32
 * inputs are computed in fp32 throughout.  Entries of idx outside [0, C) are
 * not checked on the device; they are the caller's error. */
vsa_status vsa_fine(const vsa_problem* p, const void* qcube, const void* kcube,
                    const void* vcube, const int32_t* idx, void* o_fine, float* lse,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/* The fine stage of vsa_forward on its own: raster q, k, v in, raster
 * outputs (the fine block-sparse kernel of the results section with the
 * cube gather and its inverse fused in).
 *   q, k, v       : [B,H,N,d] raster; each key cube is gathered straight
 *                   from its raster rows (bf16; fp32 returns
 *                   VSA_ERR_UNSUPPORTED).
 *   idx           : [B,H,C,topk] int32, each in [0, C), distinct per row.
 *   o_fine        : [B,H,N,d] out, raster.
 *   lse           : [B,H,Np] fp32 out in cube order, or NULL.
 *   oc, o_coarse  : optional pair (both NULL or both set): oc is a per-cube
 *                   [B,H,C,d] row (vsa_coarse's O_coarse) that is written to
 *                   every valid token of its cube in o_coarse [B,H,N,d]. */
vsa_status vsa_fine_raster(const vsa_problem* p, const void* q, const void* k, const void* v,
                           const int32_t* idx, void* o_fine, float* lse, const void* oc,
                           void* o_coarse, hipStream_t stream);

/* Dense attention: the full softmax attention that the fine stage replaces,
 * over every cube of the grid (the FastWan re-post's results section quotes
 * the fine kernel's speed-up over FlashAttention-3 on the same sequence).
 * The result equals vsa_fine with every cube selected; the kernel takes no
 * index list and shares each staged key block between two query cubes (128
 * query rows per workgroup).  It is the library's dense baseline.
 *   qcube, kcube, vcube : [B,H,Np,d] bf16 cube order; pad slots of kcube and
 *                         vcube are never attended to but must be finite.
 *   o                   : [B,H,Np,d] out, cube order (pad rows unspecified).
 *   lse                 : [B,H,Np] fp32 out (natural log), or NULL.
 * p->topk must be valid (1..C) and is not used.  VSA_F32 problems return
 * VSA_ERR_UNSUPPORTED. */
vsa_status vsa_dense(const vsa_problem* p, const void* qcube, const void* kcube,
                     const void* vcube, void* o, float* lse, hipStream_t stream);

/* Whole forward on raster tensors: reorder + coarse + fine + inverse reorder
 * (the drop-in for FlashAttention of the section on why sparse attention
 * fails under distillation).
 *   q, k, v   : [B,H,N,d] raster.
 *   o_fine    : [B,H,N,d] out, raster.
 *   o_coarse  : [B,H,N,d] out, raster; token r holds its cube's coarse row.
 *   idx       : [B,H,C,topk] int32 out, ascending (as vsa_coarse).
 *   lse       : [B,H,Np] fp32 out in cube order (for vsa_backward), or NULL.
 *   means     : [3,B,H,C,d] fp32 out, the per-cube means of q, k and v over
 *               the valid slots (the pooled operands of the coarse stage), or
 *               NULL.  Handing them to vsa_backward spares it a pass over q,
 *               k and v; writing them costs the forward nothing extra.
 *   ws        : vsa_workspace_bytes(p, VSA_OP_FORWARD) bytes. */
vsa_status vsa_forward(const vsa_problem* p, const void* q, const void* k, const void* v,
                       void* o_fine, void* o_coarse, int32_t* idx, float* lse, float* means,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* vsa_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Arguments, results and errors are
 * those of vsa_forward; the same kernels run.  Its workspace is a 32 MiB
 * device array inside the library (one per GPU, held until the process
 * ends): a problem whose vsa_workspace_bytes(p, VSA_OP_FORWARD) exceeds
 * 32 MiB returns VSA_ERR_WORKSPACE before anything is enqueued (the Wan-1.3B
 * 480p shape needs 2.4 MB; the Wan-14B 720p shape, 103 MB, does not fit).
 * The call allocates nothing: the first call on a device looks up the
 * array's device address (VSA_ERR_LAUNCH if that fails).  Every call on a
 * device uses the same array, so calls that overlap in time on one device
 * (for example on two streams) race; every byte of it a call reads is
 * written earlier in the same call. */
vsa_status vsa_forward_static(const vsa_problem* p, const void* q, const void* k,
                              const void* v, void* o_fine, void* o_coarse, int32_t* idx,
                              float* lse, float* means, hipStream_t stream);

/* Backward of vsa_forward, the trainable path (VSA trains in place of
 * FlashAttention, section on why sparse attention fails under
 * distillation).  Gradients of  sum(o_fine*do_fine) + sum(o_coarse*do_coarse)
 * w.r.t. q, k, v with the selection idx held constant:
 *   fine:   P = exp(S - lse), D = rowsum(do_fine * o_fine),
 *           dS = P * (do_fine V^T - D), dQ = dS K / sqrt(d),
 *           dK = sum over query cubes selecting the key cube of dS^T Q / sqrt(d),
 *           dV = the same sum of P^T do_fine;
 *   coarse: dOc = sum of do_coarse over each cube's valid tokens,
 *           dVc = Pc^T dOc, dSc = Pc * (dOc Vc^T - rowsum(.)),
 *           dQc = dSc Kc / sqrt(d), dKc = dSc^T Qc / sqrt(d); every valid token
 *           of a cube receives that cube's gradient divided by its valid count.
 *   q, k, v, o_fine, do_fine, do_coarse : [B,H,N,d] raster (do_coarse may be
 *           NULL, meaning zero); lse [B,H,Np] and idx as written by vsa_forward.
 *   means : [3,B,H,C,d] fp32 as written by vsa_forward for the same q, k, v,
 *           or NULL: then the means are recomputed from q, k and v.  Only the
 *           coarse gradients use them (ignored when do_coarse is NULL).
 *   dq, dk, dv : [B,H,N,d] raster out (overwritten).
 * Deterministic: no floating-point atomics; repeated calls give the same bits.
 * Implemented for VSA_BF16 (C <= 4096 cubes, as every entry point); other problems return
 * VSA_ERR_UNSUPPORTED before anything is enqueued. */
vsa_status vsa_backward(const vsa_problem* p, const void* q, const void* k, const void* v,
                        const void* o_fine, const float* lse, const int32_t* idx,
                        const float* means, const void* do_fine, const void* do_coarse,
                        void* dq, void* dk, void* dv,
                        void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- cube order kept across calls --------------------------------------
 * VSA drops in for FlashAttention inside a DiT (section on why sparse
 * attention fails under distillation): a model that keeps its tokens in cube
 * order from layer to layer calls these instead of vsa_forward/vsa_backward
 * and pays no reorder on either side.  O_coarse stays one row per cube
 * ([B,H,C,d], the row every token of the cube would receive); how it is
 * combined with O_fine is left to the caller, as for the raster calls. */

/* Whole forward on cube-order tensors.
 *   qcube, kcube, vcube : [B,H,Np,d] cube order; pad slots must be finite
 *                         (vsa_reorder writes zeros) and are never attended to.
 *   o_fine              : [B,H,Np,d] out, cube order (pad rows unspecified).
 *   o_coarse            : [B,H,C,d] out, one row per cube.
 *   idx, lse, means     : as vsa_forward.
 *   ws                  : vsa_workspace_bytes(p, VSA_OP_FORWARD_CUBE) bytes.
 * Equals vsa_forward followed by vsa_reorder of o_fine (bf16 and fp32). */
vsa_status vsa_forward_cube(const vsa_problem* p, const void* qcube, const void* kcube,
                            const void* vcube, void* o_fine, void* o_coarse, int32_t* idx,
                            float* lse, float* means, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* Backward of vsa_forward_cube: gradients of
 * sum(o_fine*do_fine) + sum(o_coarse*do_coarse) w.r.t. qcube, kcube, vcube with
 * idx held constant (the definitions of vsa_backward, with dOc = do_coarse).
 *   qcube, kcube, vcube, o_fine, do_fine : [B,H,Np,d] cube order (pad slots finite).
 *   do_coarse : [B,H,C,d], one row per cube, or NULL (zero).
 *   lse, idx  : as written by vsa_forward_cube; means as written by it, or NULL.
 *   dq, dk, dv: [B,H,Np,d] out, cube order, zero on pad slots.
 *   ws        : vsa_workspace_bytes(p, VSA_OP_BACKWARD_CUBE) bytes.
 * Limits of vsa_backward (VSA_BF16). */
vsa_status vsa_backward_cube(const vsa_problem* p, const void* qcube, const void* kcube,
                             const void* vcube, const void* o_fine, const float* lse,
                             const int32_t* idx, const float* means, const void* do_fine,
                             const void* do_coarse, void* dq, void* dk, void* dv, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* ---- FP8 fine stage ----------------------------------------------------
 * The pages note that sparse attention and low-bit attention are orthogonal
 * and stack (TurboDiffusion write-up on qq8o.cn, section "主要技术"); they
 * give no FP8 scheme for VSA.  The one below is this library's own, for
 * inference with bf16 q, k, v and d = 128 (other problems return
 * VSA_ERR_UNSUPPORTED).
 *   Codes: OCP E4M3 (bias 7, largest finite 448), round to nearest even.
 *   Scales: every (batch, head, cube) of each of q, k, v has an exponent e,
 *     the smallest integer with amax <= 448 * 2^e (amax = largest |x| over
 *     the cube's valid slots), floored at -120; the code stores x * 2^-e.
 *   Fine stage: S from the codes times 2^(eq + ek) / sqrt(d) (fp32),
 *     P = exp(S - running max) rounded to E4M3, O = sum P 2^ev V_code / sum P
 *     with fp32 accumulation; the only rounding beyond the input codes is
 *     that of P (3 mantissa bits). */

/* Quantizes bf16 raster q, k, v [B,H,N,128] into the FP8 layout:
 *   q8, k8 : [B,H,Np,128] bytes, cube order, pad slots 0.
 *   vt8    : [B,H,C,128,64] bytes: per cube the transposed V tile; byte
 *            16g + 4b + j of row dd holds key slot 16b + 4g + j of the cube
 *            (g, b, j in 0..3), the operand order of the fine kernel.
 *   exps   : int32 [3][B,H,C], the exponents e of q, k and v.
 * Bit-exact (integer exponent logic and round-to-nearest-even codes). */
vsa_status vsa_quantize_fp8(const vsa_problem* p, const void* q, const void* k, const void* v,
                            void* q8, void* k8, void* vt8, int32_t* exps, hipStream_t stream);

/* Fine stage on the FP8 layout of vsa_quantize_fp8 (the fine block-sparse
 * kernel of the FastWan re-post's results section, on E4M3 operands).
 *   idx    : [B,H,C,topk] int32, each in [0, C), distinct per row.
 *   o_fine : [B,H,Np,128] bf16 out, cube order (pad rows unspecified).
 *   lse    : [B,H,Np] fp32 out (natural log), or NULL. */
vsa_status vsa_fine_fp8(const vsa_problem* p, const void* q8, const void* k8, const void* vt8,
                        const int32_t* exps, const int32_t* idx, void* o_fine, float* lse,
                        hipStream_t stream);

/* Whole forward with the FP8 fine stage: one pass quantizes q, k, v and
 * pools the fp32 cube means, the coarse stage and the selection are those of
 * vsa_forward (fp32, exact top-K), and the fine stage runs on E4M3.
 * Arguments as vsa_forward; ws of vsa_workspace_bytes(p, VSA_OP_FORWARD_FP8). */
vsa_status vsa_forward_fp8(const vsa_problem* p, const void* q, const void* k, const void* v,
                           void* o_fine, void* o_coarse, int32_t* idx, float* lse,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* Static string naming a status. */
const char* vsa_status_string(vsa_status s);

#ifdef __cplusplus
}  /* extern "C" */
#endif
#endif  /* VSA_H_ */
