"""GPU parity of the FP8 fine stage against the oracle, through the C ABI.

Quantization (vsa_quantize_fp8) is integer exponent logic plus
round-to-nearest-even codes: it must match the oracle bit for bit.

The fine stage (vsa_fine_fp8) is compared with the oracle's exact attention
over the dequantized inputs, row by row, against bounds derived from the
kernel's arithmetic:
  * The probabilities P' (relative to the kernel's running maximum, so the
    largest is in [1, 2^8]) are rounded to E4M3 before the PV product and the
    row sum, both of which use the rounded values.  A normal value moves by at
    most 2^-4 of itself, one below 2^-6 by at most 2^-10 (half the subnormal
    step).  With P_k = exp(s_k - max s) (so P' >= P), l = sum P and
    n_sub = #{k: P_k < 2^-6}, the rounded sum moves by at most
    delta * l with delta = 2^-4 + 2^-10 n_sub / l.
  * The output is then a convex combination of the row's dequantized V rows
    whose weights move by at most 2 delta / (1 - delta) in l1 norm (and by
    at most 2 in any case).
  * The scores carry the accumulation error of the E4M3 matrix product.  The
    products of two E4M3 values are exact in fp32 (4 + 4 significant bits);
    how the matrix core sums them is not documented, so the bound assumes
    only that the sum loses at most 2^-8 of sum_d |q_d k_d| -- no worse than
    rounding the sum once to bfloat16, the precision of the inputs the path
    starts from.  No figure measured on the device enters the bound.  This
    gives ds = 2^-8 max_k sum_d |q_d k_d| / sqrt(d), which moves the weights
    by at most a factor exp(2 ds).
So per row, with vmax = max |V| over the row's selected key slots,
  |dO| <= vmax (2 delta / (1 - delta) + 2 ds + 2^-10)   (PV accumulation)
  |d lse| <= -ln(1 - delta) + ds + 2^-22 |lse|            (fp32 rounding)
The typical error is far below these bounds (the rounding errors are
unbiased and spread over many keys); the tests print the largest and the
mean error relative to vmax.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import block_sparse_attention_cube_amd as vsa
from oracle import vsa_oracle as vo
from parity import assert_close, check_idx
from synth import configs, inputs
from synth.configs import Workload

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    configs.WAN_1_3B,
    Workload("ragged-fp8-odd-k", B=2, H=3, T=5, Hh=6, Ww=7, d=128, dtype="bf16", topk=3,
             structure="offset", alpha=0.5),
    Workload("one-token-fp8", B=1, H=2, T=1, Hh=1, Ww=1, d=128, dtype="bf16", topk=1,
             structure="offset", alpha=0.5),
    Workload("all-cubes-fp8", B=1, H=2, T=8, Hh=12, Ww=10, d=128, dtype="bf16", topk=18,
             structure="field", alpha=0.5),
    Workload("one-cube-each-fp8", B=1, H=2, T=8, Hh=12, Ww=10, d=128, dtype="bf16", topk=1,
             structure="field", alpha=0.5),
    # 130 selected cubes: more than 64 steps' worth of key lists per query cube
    Workload("long-list-fp8", B=1, H=1, T=24, Hh=24, Ww=24, d=128, dtype="bf16", topk=130,
             structure="field", alpha=0.5),
]
ids = lambda ws: [w.name for w in ws]
ACC_ERR = 2.0 ** -8      # assumed accumulation error of the E4M3 product, relative to sum |a b|


def row_bounds(qdeq, kdeq, vdeq, idx, g, qcubes=None):
    """Per query row (cube order): (delta, ds, vmax) of the bounds above; NaN
    outside the valid rows of the checked cubes."""
    B, H, Np, d = qdeq.shape
    out = np.full((3, B, H, Np), np.nan)
    cubes = range(g["C"]) if qcubes is None else qcubes
    for b in range(B):
        for h in range(H):
            for i in cubes:
                rows = np.arange(64 * i, 64 * i + 64)
                rows = rows[g["valid"][rows]]
                keys = np.concatenate([np.arange(64 * j, 64 * j + 64) for j in idx[b, h, i]])
                keys = keys[g["valid"][keys]]
                q, k = qdeq[b, h, rows], kdeq[b, h, keys]
                s = q @ k.T / np.sqrt(d)
                P = np.exp(s - s.max(axis=1, keepdims=True))
                lsum = P.sum(axis=1)
                out[0, b, h, rows] = 2.0 ** -4 + 2.0 ** -10 * (P < 2.0 ** -6).sum(axis=1) / lsum
                out[1, b, h, rows] = ACC_ERR * (np.abs(q) @ np.abs(k).T).max(axis=1) / np.sqrt(d)
                out[2, b, h, rows] = np.abs(vdeq[b, h, keys]).max()
    return out


def dequantized(quant):
    return [vo.e4m3_decode(c) * np.repeat(np.ldexp(1.0, e), 64, axis=-1)[..., None] for c, e in quant]


def grid(w):
    return (w.T, w.Hh, w.Ww)


def scaled_inputs(w, seed=0):
    """The workload's inputs with every cube of v multiplied by a power of two
    between 2^-12 and 2^12 and every cube of q and k by one between 2^-2 and
    2^2, so that the cube exponents vary widely inside one head (the q, k
    range stays moderate: wider factors only make the softmax one-hot)."""
    x = inputs.make_inputs(w, seed=seed)
    g = vo.geometry(w.T, w.Hh, w.Ww)
    rng = np.random.default_rng(seed + 99)
    cube_of = g["cube_of_token"]
    for n, span in (("q", 2), ("k", 2), ("v", 12)):
        f = 2.0 ** rng.integers(-span, span + 1, size=(w.B, w.H, g["C"]))
        x[n] = (x[n] * f[..., cube_of, None]).astype(np.float32)
    return x


def expected_vt8(codes_cube, C):
    """The documented V tile layout: byte 16g + 4b + j of row dd of a cube's
    tile holds key slot 16b + 4g + j."""
    B, H, Np, d = codes_cube.shape
    t = codes_cube.reshape(B, H, C, 64, d)           # [.., key slot, dd]
    pos = np.empty(64, dtype=np.int64)               # byte position -> key slot
    for g_ in range(4):
        for b in range(4):
            for j in range(4):
                pos[16 * g_ + 4 * b + j] = 16 * b + 4 * g_ + j
    return np.swapaxes(t[..., pos, :], -1, -2)       # [.., dd, byte]


def check_fine(o, lse, ref_o, ref_lse, quant, idx, g, what, pos=None):
    """o, lse: GPU results in cube order (numpy); pos: the cube-order rows to
    check (default: every valid row)."""
    qdeq, kdeq, vdeq = dequantized(quant)
    qcubes = None if pos is None else sorted(set((pos // 64).tolist()))
    delta, ds, vmax = row_bounds(qdeq, kdeq, vdeq, idx, g, qcubes)
    rows = np.flatnonzero(g["valid"]) if pos is None else pos
    o = np.asarray(o, dtype=np.float64)[..., rows, :]
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    delta, ds, vmax = delta[..., rows], ds[..., rows], vmax[..., rows]
    err = np.abs(o - ref_o[..., rows, :]).max(axis=-1)
    # both outputs are convex combinations of the same V rows: |dO| <= 2 vmax always
    wmove = np.where(delta < 0.5, 2 * delta / (1 - np.minimum(delta, 0.5)), 2.0)
    tol = vmax * (wmove + 2 * ds + 2.0 ** -10)
    assert np.all(err <= tol), (what, "O", float((err / tol).max()))
    rel = np.abs(o - ref_o[..., rows, :]).mean(axis=-1) / vmax
    mean = rel.mean(axis=-1)                     # per (b, h), reported only
    if lse is not None:
        dl = np.abs(np.asarray(lse)[..., rows] - ref_lse[..., rows])
        tl = np.where(delta < 1, -np.log1p(-np.minimum(delta, 0.999)), np.inf) + ds \
            + 2.0 ** -22 * np.abs(ref_lse[..., rows])
        assert np.all(dl <= tl), (what, "lse", float((dl / tl).max()))
    return float((err / vmax).max()), float(mean.max())


@pytest.mark.parametrize("scaled", [False, True], ids=["plain", "scaled-cubes"])
@pytest.mark.parametrize("w", CASES[:4], ids=ids(CASES[:4]))
def test_quantize_fp8_is_bit_exact(w, scaled):
    x = scaled_inputs(w) if scaled else inputs.make_inputs(w, seed=0)
    q, k, v = (inputs.as_torch(x[n], w.dtype, DEV) for n in "qkv")
    q8, k8, vt8, exps = vsa.quantize_fp8(q, k, v, grid(w))
    torch.cuda.synchronize()
    g = vo.geometry(w.T, w.Hh, w.Ww)
    for i, (n, got) in enumerate((("q", q8), ("k", k8), ("v", vt8))):
        codes, e, _ = vo.quantize_cubes_fp8(vo.reorder(x[n].astype(np.float64), g), g)
        assert np.array_equal(exps[i].cpu().numpy(), e), f"{n}: exponents differ"
        want = expected_vt8(codes, g["C"]) if n == "v" else codes
        got = got.cpu().numpy()
        bad = np.flatnonzero(got.ravel() != want.ravel())
        assert bad.size == 0, f"{n}: {bad.size} codes differ, first at {bad[:5]}"


@pytest.mark.parametrize("scaled", [False, True], ids=["plain", "scaled-cubes"])
@pytest.mark.parametrize("w", CASES, ids=ids(CASES))
def test_fine_fp8_against_oracle(w, scaled):
    x = scaled_inputs(w) if scaled else inputs.make_inputs(w, seed=0)
    q, k, v = (inputs.as_torch(x[n], w.dtype, DEV) for n in "qkv")
    g = vo.geometry(w.T, w.Hh, w.Ww)
    qc, kc, vc = (vo.reorder(x[n].astype(np.float64), g) for n in "qkv")
    sc, _, _ = vo.coarse(vo.pool(qc, g), vo.pool(kc, g), vo.pool(vc, g))
    idx = vo.topk(sc, w.topk)
    q8, k8, vt8, exps = vsa.quantize_fp8(q, k, v, grid(w))
    o, lse = vsa.fine_fp8(q8, k8, vt8, exps, torch.from_numpy(idx.astype(np.int32)).to(DEV),
                          grid(w))
    torch.cuda.synchronize()
    ref_o, ref_lse, quant = vo.fine_fp8(qc, kc, vc, idx, g)
    mx, mean = check_fine(o.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_lse, quant, idx,
                          g, w.name)
    print(f"{w.name} scaled={scaled}: max|dO|/max|V| {mx:.4f}, mean {mean:.5f}")


@pytest.mark.parametrize("w", [configs.WAN_1_3B, CASES[1]], ids=ids([configs.WAN_1_3B, CASES[1]]))
def test_forward_fp8_end_to_end(w):
    x = inputs.make_inputs(w, seed=0)
    q, k, v = (inputs.as_torch(x[n], w.dtype, DEV) for n in "qkv")
    o_fine, o_coarse, idx, lse = vsa.forward_fp8(q, k, v, grid(w), w.topk)
    torch.cuda.synchronize()
    ref = vo.forward(x["q"], x["k"], x["v"], w.T, w.Hh, w.Ww, w.topk)
    gidx = idx.cpu().numpy()
    check_idx(gidx, ref["idx"], ref["scores"], w.topk)
    assert_close(o_coarse.float().cpu().numpy(), ref["o_coarse"], w.dtype, "O_coarse")
    g = ref["geometry"]
    qc, kc, vc = (vo.reorder(x[n].astype(np.float64), g) for n in "qkv")
    ref_o, ref_lse, quant = vo.fine_fp8(qc, kc, vc, gidx, g)
    # o_fine is raster: compare in cube order
    o_cube = vo.reorder(o_fine.float().cpu().numpy().astype(np.float64), g)
    mx, mean = check_fine(o_cube, lse.cpu().numpy(), ref_o, ref_lse, quant, gidx, g, w.name)
    # against the unquantized forward, for the record (input rounding included)
    err = np.abs(o_fine.float().cpu().numpy() - ref["o_fine"])
    print(f"{w.name}: fp8 vs oracle-on-codes max {mx:.4f} mean {mean:.5f} (of max|V|); "
          f"vs exact bf16-input forward max {err.max():.4f} mean {err.mean():.5f}")


def test_forward_fp8_wan14b_sampled():
    """Wan-14B 720p at full size; the oracle checks 4 sampled heads (whole
    coarse stage and quantization) and 16 query cubes of each."""
    w = configs.WAN_14B
    x = inputs.make_inputs(w, seed=0)
    q, k, v = (inputs.as_torch(x[n], w.dtype, DEV) for n in "qkv")
    o_fine, o_coarse, idx, lse = vsa.forward_fp8(q, k, v, grid(w), w.topk)
    torch.cuda.synchronize()
    heads, qcubes = inputs.sample_plan(w)
    hs = torch.tensor(heads, device=DEV)
    sub = {n: x[n][:, heads] for n in "qkv"}
    del x, q, k, v
    gidx = idx[:, hs].cpu().numpy()
    ref = vo.forward(sub["q"], sub["k"], sub["v"], w.T, w.Hh, w.Ww, w.topk, qcubes=qcubes)
    check_idx(gidx, ref["idx"], ref["scores"], w.topk)
    g = ref["geometry"]
    qc, kc, vc = (vo.reorder(sub[n].astype(np.float64), g) for n in "qkv")
    ref_o, ref_lse, quant = vo.fine_fp8(qc, kc, vc, gidx, g, qcubes=qcubes)
    pos = np.concatenate([np.arange(64 * c, 64 * c + 64) for c in qcubes])
    pos = pos[g["valid"][pos]]
    toks = g["token"][pos]
    o_cube = np.zeros(ref_o.shape)
    o_cube[:, :, pos] = o_fine[:, hs].float().cpu().numpy()[:, :, toks]
    mx, mean = check_fine(o_cube, lse[:, hs].cpu().numpy(), ref_o, ref_lse, quant, gidx, g,
                          "wan14b sampled", pos=pos)
    print(f"wan14b sampled: max|dO|/vmax {mx:.4f}, mean {mean:.5f}")
    assert_close(o_coarse[:, hs].float().cpu().numpy(), ref["o_coarse"], w.dtype,
                 "O_coarse sampled heads")
