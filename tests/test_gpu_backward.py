"""GPU parity of the backward (dq, dk, dv through the fine and coarse stages,
selection held constant) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import block_sparse_attention_cube_amd as vsa
from oracle import vsa_oracle as vo
from parity import assert_close
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
]
CASES = list(configs.SWEEP) + EDGE
ids = [w.name for w in CASES]


def grid(w):
    return (w.T, w.Hh, w.Ww)


def run(w, with_coarse=True):
    x = inputs.make_inputs(w, seed=0, grads=True)
    t = {n: inputs.as_torch(a, w.dtype, DEV) for n, a in x.items()}
    o_fine, o_coarse, idx, lse = vsa.forward(t["q"], t["k"], t["v"], grid(w), w.topk)
    doc = t["do_coarse"] if with_coarse else None
    dq, dk, dv = vsa.backward(t["q"], t["k"], t["v"], o_fine, lse, idx, t["do_fine"], doc, grid(w))
    torch.cuda.synchronize()
    return x, t, (o_fine, o_coarse, idx, lse), (dq, dk, dv)


@pytest.mark.parametrize("w", CASES, ids=ids)
def test_backward_matches_oracle(w):
    x, _, (_, _, idx, _), grads = run(w)
    gidx = idx.cpu().numpy()
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


def test_backward_is_deterministic():
    w = configs.SWEEP[0]
    _, t, (o_fine, _, idx, lse), first = run(w)
    again = vsa.backward(t["q"], t["k"], t["v"], o_fine, lse, idx, t["do_fine"], t["do_coarse"],
                         grid(w))
    for a, b in zip(first, again):
        assert torch.equal(a, b)


def test_autograd_function_matches_direct_calls():
    w = EDGE[0]
    x, t, (o_fine, o_coarse, idx, lse), grads = run(w)
    q, k, v = (t[n].clone().requires_grad_(True) for n in "qkv")
    of, oc, idx2 = vsa.vsa_attention(q, k, v, grid(w), w.topk)
    assert torch.equal(of, o_fine) and torch.equal(oc, o_coarse) and torch.equal(idx2, idx)
    ((of.float() * t["do_fine"].float()).sum() + (oc.float() * t["do_coarse"].float()).sum()).backward()
    for a, b in zip((q.grad, k.grad, v.grad), grads):
        assert torch.equal(a, b)
