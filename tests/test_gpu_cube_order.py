"""GPU parity of the calls that keep cube order across layers
(vsa_forward_cube, vsa_backward_cube) against the fp64 oracle, through the C
ABI.  The oracle is written on raster tensors; cube order is its reorder, and
a per-cube O_coarse gradient dOc is the raster one spread evenly over the
cube's valid tokens (the raster backward sums them back to dOc)."""
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
    configs.SWEEP[1],   # Wan-1.3B shape, top-K 11 of 112
    Workload("cube-ragged-d128", B=2, H=2, T=5, Hh=6, Ww=7, d=128, dtype="bf16", topk=3,
             structure="offset", alpha=0.5, backward=True),
    Workload("cube-ragged-d64", B=1, H=3, T=9, Hh=3, Ww=10, d=64, dtype="bf16", topk=2,
             structure="field", alpha=0.5, backward=True),
    Workload("cube-one-token", B=1, H=1, T=1, Hh=1, Ww=1, d=128, dtype="bf16", topk=1,
             structure="offset", alpha=0.5, backward=True),
]


def grid(w):
    return (w.T, w.Hh, w.Ww)


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_cube_order_forward_and_backward(w):
    x = inputs.make_inputs(w, seed=0, grads=True)
    g = vo.geometry(w.T, w.Hh, w.Ww)
    t = {n: inputs.as_torch(x[n], w.dtype, DEV) for n in x}
    cube = {n: vsa.reorder(t[n], grid(w)) for n in ("q", "k", "v", "do_fine")}
    means = torch.empty((3, w.B, w.H, g["C"], w.d), dtype=torch.float32, device=DEV)
    o, oc, idx, lse = vsa.forward_cube(cube["q"], cube["k"], cube["v"], grid(w), w.topk,
                                       means=means)
    torch.cuda.synchronize()
    ref = vo.forward(x["q"], x["k"], x["v"], w.T, w.Hh, w.Ww, w.topk)
    gidx = idx.cpu().numpy()
    near = check_idx(gidx, ref["idx"], ref["scores"], w.topk)
    ref_g = ref if near == 0 else vo.forward(x["q"], x["k"], x["v"], w.T, w.Hh, w.Ww, w.topk,
                                             idx=gidx)
    valid = g["valid"]
    assert_close(o.float().cpu().numpy(), ref_g["o_fine_cube"], w.dtype, "O_fine cube", rows=valid)
    assert_close(oc.float().cpu().numpy(), ref["oc"], w.dtype, "O_coarse per cube")
    assert_close(lse.cpu().numpy()[..., None], ref_g["lse_cube"][..., None], w.dtype, "LSE",
                 rows=valid)
    # the raster forward's O_fine, reordered, is the same tensor bit for bit
    of_r, _, _, _ = vsa.forward(t["q"], t["k"], t["v"], grid(w), w.topk)
    assert torch.equal(vsa.reorder(of_r, grid(w))[..., torch.from_numpy(valid).to(DEV), :],
                       o[..., torch.from_numpy(valid).to(DEV), :])

    # backward with a per-cube dO_coarse (a bf16 [B,H,C,d] drawn from the recipe's stream)
    # (means recomputed from the inputs, then the forward's means handed over)
    doc = inputs.as_torch(x["do_coarse"][:, :, :g["C"]], w.dtype, DEV).contiguous()
    doc64 = doc.double().cpu().numpy()
    spread = doc64[:, :, g["cube_of_token"], :] / g["n_valid"][g["cube_of_token"]][:, None]
    want = vo.backward(x["q"], x["k"], x["v"], x["do_fine"], spread, w.T, w.Hh, w.Ww, gidx)
    for m in (None, means):
        dq, dk, dv = vsa.backward_cube(cube["q"], cube["k"], cube["v"], o, lse, idx,
                                       cube["do_fine"], doc, grid(w), means=m)
        torch.cuda.synchronize()
        for name, got, ref_r in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
            gc = got.float().cpu().numpy()
            assert_close(gc, vo.reorder(ref_r, g), w.dtype, f"{name} cube order", rows=valid)
            assert np.all(gc[..., ~valid, :] == 0), f"{name}: pad rows are not zero"
