"""The forward and backward captured into HIP graphs (as bench.py times them)
and replayed: every replay, with other eager work and synchronisations in
between, must give the eager results bit for bit (the kernels are
deterministic and enqueue no memset)."""
import pytest
import torch

import block_sparse_attention_cube_amd as vsa
from synth import configs, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def tensors(w, seed):
    x = inputs.make_inputs(w, seed=seed, grads=True)
    return {n: inputs.as_torch(a, w.dtype, DEV) for n, a in x.items()}


@pytest.mark.parametrize("w", [configs.SWEEP[2], configs.WAN_1_3B],
                         ids=[configs.SWEEP[2].name, configs.WAN_1_3B.name])
def test_graph_replays_equal_eager_calls(w):
    grid = (w.T, w.Hh, w.Ww)
    t, other = tensors(w, 0), tensors(w, 1)
    fwd = vsa.ForwardPlan(w.B, w.H, grid, w.d, w.topk, torch.bfloat16, DEV, keep_means=True)
    bwd = vsa.BackwardPlan(w.B, w.H, grid, w.d, w.topk, torch.bfloat16, DEV)

    def forward_call():
        return fwd.run(t["q"], t["k"], t["v"])

    of, oc, idx, lse = (x.clone() for x in forward_call())
    means = fwd.means.clone()

    def backward_call():
        return bwd.run(t["q"], t["k"], t["v"], of, lse, idx, t["do_fine"], t["do_coarse"],
                       means=means)

    want_f = [x.clone() for x in (of, oc, idx, lse, means)]
    want_b = [x.clone() for x in backward_call()]
    torch.cuda.synchronize()

    graphs = []
    for fn in (forward_call, backward_call):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        graphs.append(graph)

    for rep in range(3):
        # eager work on other inputs between replays overwrites the plans' buffers
        fwd.run(other["q"], other["k"], other["v"])
        bwd.run(other["q"], other["k"], other["v"], of, lse, idx, other["do_fine"],
                other["do_coarse"])
        torch.cuda.synchronize()
        graphs[0].replay()
        torch.cuda.synchronize()
        got_f = (fwd.o_fine, fwd.o_coarse, fwd.idx, fwd.lse, fwd.means)
        for name, a, b in zip(("o_fine", "o_coarse", "idx", "lse", "means"), got_f, want_f):
            assert torch.equal(a, b), f"forward replay {rep}: {name}"
        graphs[1].replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), (bwd.dq, bwd.dk, bwd.dv), want_b):
            assert torch.equal(a, b), f"backward replay {rep}: {name}"
