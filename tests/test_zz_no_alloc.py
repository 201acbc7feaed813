"""vsa_forward_static (the forward that allocates nothing: its workspace is a
device array inside the library) against vsa_forward, through the C ABI.
Both run the same kernels, so the results must be bit-identical.  Two calls
in a row, the second on a smaller problem, so that the second must not read
anything the first left in the shared array."""
import ctypes

import pytest
import torch

import block_sparse_attention_cube_amd as vsa
from block_sparse_attention_cube_amd import _lib as L
from synth import configs, inputs
from synth.configs import Workload

pytestmark = pytest.mark.gpu
DEV = "cuda"

SMALLER = Workload("ragged-static", B=2, H=3, T=5, Hh=6, Ww=7, d=128, dtype="bf16", topk=3,
                   structure="offset", alpha=0.5)


def outputs_like(w):
    C, Np = vsa.cube_counts((w.T, w.Hh, w.Ww))
    shape = (w.B, w.H, w.N, w.d)
    return (torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV),
            torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV),
            torch.full((w.B, w.H, C, w.topk), -1, dtype=torch.int32, device=DEV),
            torch.full((w.B, w.H, Np), float("nan"), dtype=torch.float32, device=DEV))


def test_static_forward_equals_forward_on_two_calls():
    for w in (configs.WAN_1_3B, SMALLER):
        grid = (w.T, w.Hh, w.Ww)
        x = inputs.make_inputs(w, seed=0)
        q, k, v = (inputs.as_torch(x[n], w.dtype, DEV) for n in "qkv")
        want = [t.clone() for t in vsa.forward(q, k, v, grid, w.topk)]
        out = outputs_like(w)
        got = vsa.forward_static(q, k, v, grid, w.topk, out=out)
        torch.cuda.synchronize()
        for name, a, b in zip(("o_fine", "o_coarse", "idx", "lse"), got, want):
            assert torch.equal(a, b), f"{w.name}: {name} differs from vsa_forward"


def test_static_forward_rejects_problems_beyond_its_scratch():
    w = configs.WAN_14B       # 103 MB of workspace, beyond the 32 MiB array
    p = vsa.make_problem(w.B, w.H, (w.T, w.Hh, w.Ww), w.d, w.topk, torch.bfloat16)
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: the size check comes first
    st = L.lib().vsa_forward_static(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None,
                                    None, None)
    assert st == L.VSA_ERR_WORKSPACE
