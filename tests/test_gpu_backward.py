"""GPU parity of the backward (dq, dk, dv through the fine and coarse stages,
selection held constant) against the fp64 oracle, through the C ABI."""
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

EDGE = [
    Workload("bwd-ragged-d128", B=2, H=2, T=5, Hh=6, Ww=7, d=128, dtype="bf16", topk=3,
             structure="offset", alpha=0.5, backward=True),
    Workload("bwd-ragged-d64", B=1, H=3, T=9, Hh=3, Ww=10, d=64, dtype="bf16", topk=2,
             structure="field", alpha=0.5, backward=True),
    Workload("bwd-all-cubes", B=1, H=2, T=8, Hh=12, Ww=10, d=128, dtype="bf16", topk=18,
             structure="field", alpha=0.5, backward=True),
    Workload("bwd-one-cube", B=1, H=2, T=8, Hh=12, Ww=10, d=128, dtype="bf16", topk=1,
             structure="field", alpha=0.5, backward=True),
    Workload("bwd-one-token", B=1, H=1, T=1, Hh=1, Ww=1, d=128, dtype="bf16", topk=1,
             structure="offset", alpha=0.5, backward=True),
    # 552 cubes: above the bitmap limit of the block-list transpose (512), so
    # the round-by-round transpose runs; ragged last cube column
    Workload("bwd-many-cubes", B=1, H=1, T=4, Hh=96, Ww=90, d=64, dtype="bf16", topk=3,
             structure="field", alpha=0.5, backward=True),
    # 1280 cubes: above 1216, the coarse backward takes 8 cubes per workgroup
    # (two 8 x C score tiles in LDS); ragged edges on both spatial axes.  The
    # per-cube offsets spread the selections (at most 12 query cubes per key
    # cube): with the smooth field one key cube collects 53 and its dv reaches
    # 9.7, where rounding the exact value to bf16 alone costs 0.0295 of the
    # 0.03 bound
    Workload("bwd-1280-cubes", B=1, H=1, T=4, Hh=126, Ww=158, d=64, dtype="bf16", topk=2,
             structure="offset", alpha=0.5, backward=True),
    # 2304 cubes: the coarse backward takes 4 cubes per workgroup
    Workload("bwd-2304-cubes", B=1, H=1, T=4, Hh=190, Ww=189, d=64, dtype="bf16", topk=2,
             structure="offset", alpha=0.5, backward=True),
    # top-K above 64: the dQ tiles reload their per-lane key table mid-walk and
    # dK/dV block lists run past 64 entries; one-frame last cube layer (its
    # waves hold time slices, three of four idle on that layer)
    Workload("bwd-t13-k70", B=1, H=1, T=13, Hh=16, Ww=24, d=64, dtype="bf16", topk=70,
             structure="field", alpha=0.5, backward=True),
]
CASES = list(configs.SWEEP) + EDGE
ids = [w.name for w in CASES]


def grid(w):
    return (w.T, w.Hh, w.Ww)


def means_like(w):
    return torch.full((3, w.B, w.H, w.C, w.d), float("nan"), dtype=torch.float32, device=DEV)


def run(w, with_coarse=True, keep_means=False):
    """Forward then backward; keep_means: the forward writes its per-cube
    means and the backward takes them instead of recomputing them."""
    x = inputs.make_inputs(w, seed=0, grads=True)
    t = {n: inputs.as_torch(a, w.dtype, DEV) for n, a in x.items()}
    means = means_like(w) if keep_means else None
    o_fine, o_coarse, idx, lse = vsa.forward(t["q"], t["k"], t["v"], grid(w), w.topk,
                                             means=means)
    doc = t["do_coarse"] if with_coarse else None
    dq, dk, dv = vsa.backward(t["q"], t["k"], t["v"], o_fine, lse, idx, t["do_fine"], doc, grid(w),
                              means=means)
    torch.cuda.synchronize()
    if keep_means:
        t["means"] = means
    return x, t, (o_fine, o_coarse, idx, lse), (dq, dk, dv)


def check_forward(w, x, outs):
    """The forward that feeds the backward, against the oracle: the selection
    by the near-tie rule, then O_fine (on the GPU's own selection), O_coarse
    and LSE element by element."""
    o_fine, o_coarse, idx, lse = outs
    gidx = idx.cpu().numpy()
    ref = vo.forward(x["q"], x["k"], x["v"], w.T, w.Hh, w.Ww, w.topk)
    near = check_idx(gidx, ref["idx"], ref["scores"], w.topk)
    ref_g = ref if near == 0 else vo.forward(x["q"], x["k"], x["v"], w.T, w.Hh, w.Ww, w.topk,
                                             idx=gidx)
    errs = {
        "o_fine": assert_close(o_fine.float().cpu().numpy(), ref_g["o_fine"], w.dtype, "O_fine"),
        "o_coarse": assert_close(o_coarse.float().cpu().numpy(), ref["o_coarse"], w.dtype,
                                 "O_coarse"),
        "lse": assert_close(lse.cpu().numpy()[..., None], ref_g["lse_cube"][..., None], w.dtype,
                            "LSE", rows=ref_g["geometry"]["valid"]),
    }
    print(f"{w.name}: near-tie rows {near}; max/mean |err| " +
          ", ".join(f"{k} {a:.2e}/{b:.2e}" for k, (a, b) in errs.items()))


@pytest.mark.parametrize("w", CASES, ids=ids)
def test_backward_matches_oracle(w):
    x, _, outs, grads = run(w)
    check_forward(w, x, outs)
    gidx = outs[2].cpu().numpy()
    ref = vo.backward(x["q"], x["k"], x["v"], x["do_fine"], x["do_coarse"], w.T, w.Hh, w.Ww, gidx)
    for name, got, want in zip(("dq", "dk", "dv"), grads, ref):
        assert_close(got.float().cpu().numpy(), want, w.dtype, name)


@pytest.mark.parametrize("w", [configs.SWEEP[1], EDGE[0]], ids=[configs.SWEEP[1].name, EDGE[0].name])
def test_backward_fine_branch_only(w):
    x, _, (_, _, idx, _), grads = run(w, with_coarse=False)
    gidx = idx.cpu().numpy()
    zero = np.zeros_like(x["do_coarse"])
    ref = vo.backward(x["q"], x["k"], x["v"], x["do_fine"], zero, w.T, w.Hh, w.Ww, gidx)
    for name, got, want in zip(("dq", "dk", "dv"), grads, ref):
        assert_close(got.float().cpu().numpy(), want, w.dtype, name)


MEANS_CASES = [configs.SWEEP[2], EDGE[0], EDGE[1]]


@pytest.mark.parametrize("w", MEANS_CASES, ids=[w.name for w in MEANS_CASES])
def test_backward_with_the_forward_means(w):
    """The forward's per-cube means (the pooled q, k, v of the coarse stage)
    against the oracle's pool, and the gradients of a backward that takes them
    instead of reading q, k, v again."""
    x, t, (_, _, idx, _), grads = run(w, keep_means=True)
    g = vo.geometry(w.T, w.Hh, w.Ww)
    for i, n in enumerate("qkv"):
        want = vo.pool(vo.reorder(np.asarray(x[n], dtype=np.float64), g), g)
        got = t["means"][i].double().cpu().numpy()
        # a mean of at most 64 bf16 values summed in fp32: each partial sum is
        # rounded once, relative 2^-24 per addition
        bound = 64 * 2.0 ** -24 * np.abs(np.asarray(x[n], dtype=np.float64)).max() + 1e-30
        assert np.abs(got - want).max() <= bound, f"{n} means"
    gidx = idx.cpu().numpy()
    ref = vo.backward(x["q"], x["k"], x["v"], x["do_fine"], x["do_coarse"], w.T, w.Hh, w.Ww, gidx)
    for name, got, want in zip(("dq", "dk", "dv"), grads, ref):
        assert_close(got.float().cpu().numpy(), want, w.dtype, name)


def test_backward_is_deterministic():
    w = configs.SWEEP[0]
    _, t, (o_fine, _, idx, lse), first = run(w)
    again = vsa.backward(t["q"], t["k"], t["v"], o_fine, lse, idx, t["do_fine"], t["do_coarse"],
                         grid(w))
    for a, b in zip(first, again):
        assert torch.equal(a, b)


def test_autograd_function_matches_direct_calls():
    # the Function hands the forward's means to its backward, as run() does here
    w = EDGE[0]
    x, t, (o_fine, o_coarse, idx, lse), grads = run(w, keep_means=True)
    q, k, v = (t[n].clone().requires_grad_(True) for n in "qkv")
    of, oc, idx2 = vsa.vsa_attention(q, k, v, grid(w), w.topk)
    assert torch.equal(of, o_fine) and torch.equal(oc, o_coarse) and torch.equal(idx2, idx)
    ((of.float() * t["do_fine"].float()).sum() + (oc.float() * t["do_coarse"].float()).sum()).backward()
    for a, b in zip((q.grad, k.grad, v.grad), grads):
        assert torch.equal(a, b)


def test_backward_wan14b_sampled():
    """Wan-14B 720p shape (1440 cubes, top-K 144) forward and backward at full
    size on the GPU; the oracle checks dq on 6 sampled query cubes and dk, dv
    on 4 sampled key cubes (with every query cube that selected them) of 2
    sampled heads, plus the whole coarse-stage gradient of those heads."""
    w = replace(configs.WAN_14B, backward=True)
    x = inputs.make_inputs(w, seed=0, grads=True)
    t = {n: inputs.as_torch(a, w.dtype, DEV) for n, a in x.items()}
    o_fine, o_coarse, idx, lse = vsa.forward(t["q"], t["k"], t["v"], grid(w), w.topk)
    dq, dk, dv = vsa.backward(t["q"], t["k"], t["v"], o_fine, lse, idx, t["do_fine"],
                              t["do_coarse"], grid(w))
    torch.cuda.synchronize()
    heads, qcubes = inputs.sample_plan(w, n_heads=2, n_qcubes=6)
    kcubes = qcubes[:2] + qcubes[-2:]
    hs = torch.tensor(heads, device=DEV)
    sub = {n: x[n][:, heads] for n in x}
    del x, t
    gidx = idx[:, hs].cpu().numpy()
    ref = vo.backward_sampled(sub["q"], sub["k"], sub["v"], sub["do_fine"], sub["do_coarse"],
                              w.T, w.Hh, w.Ww, gidx, qcubes, kcubes)
    g = vo.geometry(w.T, w.Hh, w.Ww)
    cube = g["cube_of_token"]
    for name, got, want, cubes in (("dq", dq, ref[0], qcubes), ("dk", dk, ref[1], kcubes),
                                   ("dv", dv, ref[2], kcubes)):
        toks = np.flatnonzero(np.isin(cube, cubes))
        assert_close(got[:, hs].float().cpu().numpy()[:, :, toks], want[:, :, toks], w.dtype,
                     f"{name} sampled")
