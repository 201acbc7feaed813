"""Plain fp64 CPU oracle of video sparse attention (VSA).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this file: only tests/, the smoke check in __graft_entry__.py and the
CPU-baseline leg of bench.py use it.  It shares no code, header, table or
helper with the HIP library; both sides only share the seeded input
generator (synth/), which holds none of the method's arithmetic.

What VSA computes, and where the pages state it
------------------------------------------------
* VSA is a dynamic sparse attention that finds the important tokens itself
  and drops in for FlashAttention during training (FastWan/VSA re-post on
  yumynutrition.com, section "传统零散郑重力，为何会在蒸馏中失效？"; the
  neican.ai commentary "超越Sora：FastWan如何以“稀疏蒸馏”重塑实时AI视频生成范式",
  section "技术原理与创新点解析").  So the fine stage is exact softmax
  attention, scaled by 1/sqrt(d) as the attention it replaces.
* It has a coarse stage whose output is a block-sparse attention pattern,
  and a fine block-sparse kernel working on 64x64 blocks (yumynutrition
  re-post, results section "一张卡，秒生视频": the fine-kernel speed line,
  the coarse-stage overhead line, the FlexAttention 64x64-block-mask line
  and Fig. 5).
* At 87.5% sparsity attention FLOPs drop 8x (same results section, the
  410M scaling experiment), i.e. sparsity = 1 - K/C over C key blocks.

Readings where the pages are silent:
* a 64-token block of a video token grid is a 4x4x4 cube; cubes are taken in
  raster order of the cube grid and slots inside a cube in raster order of
  (t, y, x); each axis is padded at its high end to a multiple of 4, pad
  slots are zero and are never attended to;
* the coarse stage mean-pools q, k, v over the valid slots of each cube,
  scores every query cube against every key cube with Qc Kc^T / sqrt(d),
  softmaxes each row over all cubes (O_coarse = Pc Vc), and keeps for each
  query cube the K key cubes with the largest score, ties to the lower cube
  index, listed in ascending cube order;
* O_coarse is returned per token: token r gets the row of its own cube;
* the backward treats the selection as constant; gradients reach q, k, v
  through the fine stage and through the coarse stage (the mean-pool spreads
  a cube's gradient evenly over its valid tokens).

Everything is float64 NumPy.  Loops run over (batch, head, query cube); each
iteration is a small dense problem written as its definition.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, Optional, Sequence

import numpy as np

CUBE = 4          # cube edge (tokens per axis)
SLOTS = 64        # tokens per cube


# ----------------------------------------------------------------------------
# cube geometry and the raster <-> cube permutation
# ----------------------------------------------------------------------------

def geometry(T: int, Hh: int, Ww: int) -> Dict[str, np.ndarray]:
    """Cube grid of a (T, Hh, Ww) token grid.

    token[p] is the raster index (t*Hh + y)*Ww + x of the token held by
    cube-order position p = 64*c + (it*16 + ih*4 + iw), where cube
    c = (ct*Ch + ch)*Cw + cw holds token (4ct+it, 4ch+ih, 4cw+iw); token[p] is
    -1 for a pad slot (outside the real grid).  n_valid[c] counts real slots.
    """
    Ct, Ch, Cw = -(-T // CUBE), -(-Hh // CUBE), -(-Ww // CUBE)
    C = Ct * Ch * Cw
    token = np.full(C * SLOTS, -1, dtype=np.int64)
    cube_of_token = np.empty(T * Hh * Ww, dtype=np.int64)
    for ct in range(Ct):
        for ch in range(Ch):
            for cw in range(Cw):
                c = (ct * Ch + ch) * Cw + cw
                for it in range(CUBE):
                    for ih in range(CUBE):
                        for iw in range(CUBE):
                            t, y, x = CUBE * ct + it, CUBE * ch + ih, CUBE * cw + iw
                            if t < T and y < Hh and x < Ww:
                                r = (t * Hh + y) * Ww + x
                                token[SLOTS * c + it * 16 + ih * 4 + iw] = r
                                cube_of_token[r] = c
    valid = token >= 0
    n_valid = valid.reshape(C, SLOTS).sum(axis=1)
    return {"T": T, "Hh": Hh, "Ww": Ww, "Ct": Ct, "Ch": Ch, "Cw": Cw, "C": C,
            "Np": C * SLOTS, "N": T * Hh * Ww, "token": token, "valid": valid,
            "n_valid": n_valid, "cube_of_token": cube_of_token}


def reorder(x: np.ndarray, g) -> np.ndarray:
    """Raster (..., N, d) -> cube order (..., Np, d); pad slots are zero."""
    out = np.zeros(x.shape[:-2] + (g["Np"], x.shape[-1]), dtype=np.float64)
    out[..., g["valid"], :] = x[..., g["token"][g["valid"]], :]
    return out


def inverse_reorder(xc: np.ndarray, g) -> np.ndarray:
    """Cube order (..., Np, d) -> raster (..., N, d); pad slots are dropped."""
    out = np.empty(xc.shape[:-2] + (g["N"], xc.shape[-1]), dtype=np.float64)
    out[..., g["token"][g["valid"]], :] = xc[..., g["valid"], :]
    return out


# ----------------------------------------------------------------------------
# coarse stage
# ----------------------------------------------------------------------------

def pool(xc: np.ndarray, g) -> np.ndarray:
    """Mean over the valid slots of each cube: (..., Np, d) -> (..., C, d)."""
    C = g["C"]
    blocks = xc.reshape(xc.shape[:-2] + (C, SLOTS, xc.shape[-1]))
    mask = g["valid"].reshape(C, SLOTS, 1)
    return (blocks * mask).sum(axis=-2) / g["n_valid"][:, None]


def softmax_rows(s: np.ndarray) -> np.ndarray:
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def coarse(qc: np.ndarray, kc: np.ndarray, vc: np.ndarray):
    """Cube-level attention: Sc = Qc Kc^T / sqrt(d), Pc = softmax(Sc), Oc = Pc Vc."""
    d = qc.shape[-1]
    sc = qc @ np.swapaxes(kc, -1, -2) / math.sqrt(d)
    pc = softmax_rows(sc)
    return sc, pc, pc @ vc


def topk(sc: np.ndarray, K: int) -> np.ndarray:
    """Per row, the K key cubes with the largest score, ties to the lower index,
    returned in ascending cube order (int32)."""
    lead = sc.shape[:-1]
    rows = sc.reshape(-1, sc.shape[-1])
    out = np.empty((rows.shape[0], K), dtype=np.int32)
    for i, row in enumerate(rows):
        # a stable sort on the negated score keeps equal scores in index order
        order = np.argsort(-row, kind="stable")
        out[i] = np.sort(order[:K])
    return out.reshape(lead + (K,))


# ----------------------------------------------------------------------------
# fine stage
# ----------------------------------------------------------------------------

def _key_positions(sel: Sequence[int], g) -> np.ndarray:
    """Cube-order positions of the valid slots of the selected cubes."""
    pos = np.concatenate([np.arange(SLOTS * j, SLOTS * j + SLOTS) for j in sel])
    return pos[g["valid"][pos]]


def fine(qc: np.ndarray, kc: np.ndarray, vc: np.ndarray, idx: np.ndarray, g,
         qcubes: Optional[Iterable[int]] = None):
    """Exact softmax attention of each query cube over its selected key cubes.

    qc/kc/vc are cube-order (B, H, Np, d); idx is (B, H, C, K).  Returns
    o (B, H, Np, d) and lse (B, H, Np) (natural log of the softmax
    denominator).  Rows that are pad slots, or cubes not in qcubes, are NaN.
    """
    B, H, Np, d = qc.shape
    scale = 1.0 / math.sqrt(d)
    o = np.full((B, H, Np, d), np.nan)
    lse = np.full((B, H, Np), np.nan)
    cubes = range(g["C"]) if qcubes is None else qcubes
    for b in range(B):
        for h in range(H):
            for i in cubes:
                rows = np.arange(SLOTS * i, SLOTS * i + SLOTS)
                rows = rows[g["valid"][rows]]
                keys = _key_positions(idx[b, h, i], g)
                s = qc[b, h, rows] @ kc[b, h, keys].T * scale
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                den = e.sum(axis=1, keepdims=True)
                o[b, h, rows] = (e / den) @ vc[b, h, keys]
                lse[b, h, rows] = (m + np.log(den))[:, 0]
    return o, lse


# ----------------------------------------------------------------------------
# whole forward / backward
# ----------------------------------------------------------------------------

def forward(q, k, v, T: int, Hh: int, Ww: int, K: int,
            qcubes: Optional[Iterable[int]] = None, idx: Optional[np.ndarray] = None):
    """VSA forward on raster q, k, v (B, H, N, d).

    Returns O_fine and O_coarse in raster order (B, H, N, d), the block index
    list idx (B, H, C, K), the coarse scores Sc and softmax Pc (B, H, C, C),
    the per-cube coarse output Oc (B, H, C, d) and the fine LSE in cube order.
    A given idx replaces the coarse selection (to check the fine stage on a
    mask chosen elsewhere).
    """
    g = geometry(T, Hh, Ww)
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    qcb, kcb, vcb = reorder(q, g), reorder(k, g), reorder(v, g)
    qp, kp, vp = pool(qcb, g), pool(kcb, g), pool(vcb, g)
    sc, pc, oc = coarse(qp, kp, vp)
    if idx is None:
        idx = topk(sc, K)
    o_cube, lse = fine(qcb, kcb, vcb, idx, g, qcubes)
    return {
        "o_fine": inverse_reorder(o_cube, g),
        "o_coarse": oc[..., g["cube_of_token"], :],
        "idx": idx, "scores": sc, "pc": pc, "oc": oc,
        "o_fine_cube": o_cube, "lse_cube": lse, "geometry": g,
    }


def backward(q, k, v, do_fine, do_coarse, T: int, Hh: int, Ww: int, idx: np.ndarray):
    """Gradients of sum(O_fine*do_fine) + sum(O_coarse*do_coarse) w.r.t. raster q, k, v.

    The selection idx is held constant.  Fine stage, per query cube with
    P = softmax(S), S = Q K_sel^T / sqrt(d):
        dV_sel += P^T dO,  dP = dO V_sel^T,  dS = P * (dP - rowsum(P * dP)),
        dQ = dS K_sel / sqrt(d),  dK_sel += dS^T Q / sqrt(d).
    Coarse stage, with O_coarse[r] = Oc[cube(r)]:
        dOc[c] = sum of do_coarse over the valid tokens of cube c,
        dVc = Pc^T dOc,  dPc = dOc Vc^T,  dSc = Pc * (dPc - rowsum(Pc * dPc)),
        dQc = dSc Kc / sqrt(d),  dKc = dSc^T Qc / sqrt(d),
    and each valid token of cube c receives dQc[c] / n_c (same for k, v).
    """
    g = geometry(T, Hh, Ww)
    q, k, v, dof, doc = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do_fine, do_coarse))
    B, H, _, d = q.shape
    scale = 1.0 / math.sqrt(d)
    qcb, kcb, vcb, docb = reorder(q, g), reorder(k, g), reorder(v, g), reorder(dof, g)
    dq = np.zeros_like(qcb)
    dk = np.zeros_like(kcb)
    dv = np.zeros_like(vcb)
    for b in range(B):
        for h in range(H):
            for i in range(g["C"]):
                rows = np.arange(SLOTS * i, SLOTS * i + SLOTS)
                rows = rows[g["valid"][rows]]
                keys = _key_positions(idx[b, h, i], g)
                Q, Kk, V, dO = qcb[b, h, rows], kcb[b, h, keys], vcb[b, h, keys], docb[b, h, rows]
                P = softmax_rows(Q @ Kk.T * scale)
                dP = dO @ V.T
                dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
                dq[b, h, rows] += dS @ Kk * scale
                dk[b, h, keys] += dS.T @ Q * scale
                dv[b, h, keys] += P.T @ dO
    # coarse stage
    n = g["n_valid"][:, None]
    qp, kp, vp = pool(qcb, g), pool(kcb, g), pool(vcb, g)
    _, pc, _ = coarse(qp, kp, vp)
    doc_sum = pool(reorder(doc, g), g) * n          # sum (not mean) over valid tokens
    dvc = np.swapaxes(pc, -1, -2) @ doc_sum
    dpc = doc_sum @ np.swapaxes(vp, -1, -2)
    dsc = pc * (dpc - (pc * dpc).sum(axis=-1, keepdims=True))
    dqc = dsc @ kp * scale
    dkc = np.swapaxes(dsc, -1, -2) @ qp * scale
    per_slot = lambda x: np.repeat(x / n, SLOTS, axis=-2) * g["valid"][:, None]
    dq += per_slot(dqc)
    dk += per_slot(dkc)
    dv += per_slot(dvc)
    return inverse_reorder(dq, g), inverse_reorder(dk, g), inverse_reorder(dv, g)


def backward_sampled(q, k, v, do_fine, do_coarse, T: int, Hh: int, Ww: int, idx: np.ndarray,
                     qcubes: Sequence[int], kcubes: Sequence[int]):
    """The gradients of `backward` on a sample, for shapes too large for it.

    dq is computed on the valid tokens of the query cubes `qcubes`, dk and dv
    on those of the key cubes `kcubes`; every other element is NaN.  The
    definitions are those of `backward`: a sampled key cube receives the
    contributions of every query cube whose selection holds it (each such
    query cube's softmax is taken over all of its selected keys), plus its
    share of the coarse-stage gradient, which is computed for the whole head.
    Returns raster (B, H, N, d) arrays.
    """
    g = geometry(T, Hh, Ww)
    q, k, v, dof, doc = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do_fine, do_coarse))
    B, H, _, d = q.shape
    scale = 1.0 / math.sqrt(d)
    qcb, kcb, vcb, docb = reorder(q, g), reorder(k, g), reorder(v, g), reorder(dof, g)
    qset, kset = set(int(i) for i in qcubes), set(int(j) for j in kcubes)
    cube_rows = lambda c: np.arange(SLOTS * c, SLOTS * c + SLOTS)
    sampled = lambda cubes: np.isin(np.arange(g["Np"]) // SLOTS, sorted(cubes)) & g["valid"]
    qrows, krows = sampled(qset), sampled(kset)
    dq = np.where(qrows[:, None], 0.0, np.nan) * np.ones_like(qcb)
    dk = np.where(krows[:, None], 0.0, np.nan) * np.ones_like(kcb)
    dv = dk.copy()
    for b in range(B):
        for h in range(H):
            sel = idx[b, h]
            for i in range(g["C"]):
                hit = [j for j in sel[i] if int(j) in kset]
                if i not in qset and not hit:
                    continue
                rows = cube_rows(i)
                rows = rows[g["valid"][rows]]
                keys = _key_positions(sel[i], g)
                Q, Kk, V, dO = qcb[b, h, rows], kcb[b, h, keys], vcb[b, h, keys], docb[b, h, rows]
                P = softmax_rows(Q @ Kk.T * scale)
                dP = dO @ V.T
                dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
                if i in qset:
                    dq[b, h, rows] += dS @ Kk * scale
                for j in hit:
                    cols = (keys // SLOTS) == j
                    dk[b, h, keys[cols]] += dS[:, cols].T @ Q * scale
                    dv[b, h, keys[cols]] += P[:, cols].T @ dO
    # coarse stage, whole head (C x C), added on the sampled rows
    n = g["n_valid"][:, None]
    qp, kp, vp = pool(qcb, g), pool(kcb, g), pool(vcb, g)
    _, pc, _ = coarse(qp, kp, vp)
    doc_sum = pool(reorder(doc, g), g) * n
    dvc = np.swapaxes(pc, -1, -2) @ doc_sum
    dpc = doc_sum @ np.swapaxes(vp, -1, -2)
    dsc = pc * (dpc - (pc * dpc).sum(axis=-1, keepdims=True))
    dqc = dsc @ kp * scale
    dkc = np.swapaxes(dsc, -1, -2) @ qp * scale
    per_slot = lambda x: np.repeat(x / n, SLOTS, axis=-2)
    dq += per_slot(dqc)
    dk += per_slot(dkc)
    dv += per_slot(dvc)
    nan_raster = lambda x: np.where(np.isnan(x), np.nan, x)
    return tuple(inverse_reorder(nan_raster(x), g) for x in (dq, dk, dv))


# ----------------------------------------------------------------------------
# FP8 fine stage (a design of this library, not of the pages)
# ----------------------------------------------------------------------------
# The TurboDiffusion write-up (qq8o.cn, section "方法", "主要技术") notes that
# sparse attention and low-bit attention are orthogonal and stack.  The pages
# give no FP8 scheme for VSA; the one modelled here is this library's own:
#   * q, k, v are stored in cube order as OCP E4M3 codes (1 sign bit,
#     4 exponent bits with bias 7, 3 mantissa bits; largest finite 448,
#     subnormal step 2^-9), rounded to nearest, ties to even;
#   * every (batch, head, cube) of each tensor carries its own power-of-two
#     scale 2^e: the smallest e with amax <= 448 * 2^e, where amax is the
#     largest |x| over the cube's valid slots, and never below 2^-120;
#   * the fine stage is exact softmax attention over the dequantized values
#     (code * 2^e).  The kernel additionally rounds its probabilities to E4M3;
#     that rounding is not modelled here (it depends on the kernel's running
#     maximum) and is covered by a tolerance instead.

E4M3_MAX = 448.0
E4M3_MIN_EXP = -120


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest E4M3 value, ties to even.

    Normal values (|x| >= 2^-6) keep 3 mantissa bits, i.e. a quantum of
    2^(E-3) for |x| in [2^E, 2^(E+1)); below 2^-6 the quantum is the subnormal
    step 2^-9.  Values that would round beyond 448 are an error: the scales
    above keep every scaled value within range.
    """
    x = np.asarray(x, dtype=np.float64)
    _, p = np.frexp(x)                 # |x| = m 2^p, m in [0.5, 1)
    expo = np.maximum(p - 1, -6)       # E, floored at the smallest normal exponent
    quantum = np.ldexp(1.0, expo - 3)
    y = np.round(x / quantum) * quantum   # np.round rounds halves to even
    if np.any(np.abs(y) > E4M3_MAX):
        raise ValueError("value outside the E4M3 range")
    return y


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Bit pattern (uint8) of values that are already E4M3 values."""
    y = np.asarray(y, dtype=np.float64)
    sign = (np.signbit(y)).astype(np.uint8) << 7
    a = np.abs(y)
    _, p = np.frexp(a)
    e = p - 1                                          # a in [2^e, 2^(e+1))
    normal = a >= 2.0 ** -6
    exp_field = np.where(normal, e + 7, 0)
    mant = np.where(normal, a / np.ldexp(1.0, e) - 1.0, a / 2.0 ** -9 / 8.0) * 8.0
    mant = np.where(a == 0, 0, mant)
    exp_field = np.where(a == 0, 0, exp_field)
    code = (exp_field.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    return sign | code.astype(np.uint8)


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """Value of E4M3 bit patterns (the all-ones exponent/mantissa pattern is NaN)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef, mf = (c >> 3) & 15, c & 7
    mag = np.where(ef == 0, mf * 2.0 ** -9, np.ldexp(1.0 + mf / 8.0, ef - 7))
    mag = np.where((ef == 15) & (mf == 7), np.nan, mag)
    return sign * mag


def fp8_scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e, floored at -120."""
    a = np.asarray(amax, dtype=np.float64)
    m, p = np.frexp(a)                  # a = m 2^p; 448 = 1.75 * 2^8
    f, big_e = 2.0 * m, p - 1          # a = f 2^E, f in [1, 2)
    e = np.where(f <= 1.75, big_e - 8, big_e - 7)
    e = np.where(a == 0, E4M3_MIN_EXP, e)
    return np.maximum(e, E4M3_MIN_EXP).astype(np.int64)


def quantize_cubes_fp8(xc: np.ndarray, g):
    """Per-cube E4M3 quantization of a cube-order tensor (..., Np, d).

    Returns (codes uint8 (..., Np, d), exponents int64 (..., C), dequantized
    float64 (..., Np, d)).  Pad slots are zero in all three.
    """
    xc = np.asarray(xc, dtype=np.float64)
    lead, Np, d = xc.shape[:-2], xc.shape[-2], xc.shape[-1]
    cubes = xc.reshape(*lead, Np // SLOTS, SLOTS, d)
    valid = g["valid"].reshape(Np // SLOTS, SLOTS)[..., None]
    amax = np.abs(np.where(valid, cubes, 0.0)).max(axis=(-2, -1))
    e = fp8_scale_exponent(amax)
    scale = np.ldexp(1.0, e)[..., None, None]
    y = e4m3_round(np.where(valid, cubes, 0.0) / scale)
    deq = (y * scale).reshape(xc.shape)
    return e4m3_encode(y).reshape(xc.shape), e, deq


def fine_fp8(qc: np.ndarray, kc: np.ndarray, vc: np.ndarray, idx: np.ndarray, g,
             qcubes: Optional[Iterable[int]] = None):
    """Fine stage on E4M3-quantized q, k, v (cube order): exact attention over
    the dequantized values.  Returns o, lse and the per-tensor
    (codes, exponents) of the quantization."""
    quant = [quantize_cubes_fp8(x, g) for x in (qc, kc, vc)]
    o, lse = fine(quant[0][2], quant[1][2], quant[2][2], idx, g, qcubes)
    return o, lse, [(c, e) for c, e, _ in quant]
