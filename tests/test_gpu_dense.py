"""GPU parity of the dense baseline (vsa_dense: attention over every cube,
no index list) against the fp64 oracle's fine stage with every cube
selected, through the C ABI."""
import numpy as np
import pytest
import torch

import block_sparse_attention_cube_amd as vsa
from oracle import vsa_oracle as vo
from parity import assert_close
from synth import inputs
from synth.configs import Workload

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # the Wan-1.3B 480p grid (112 cubes, pad keys in its edge cubes), 2 heads
    Workload("dense-wan1.3b-h2", B=1, H=2, T=16, Hh=14, Ww=26, d=128, dtype="bf16", topk=112,
             structure="field", alpha=0.5),
    # its 5824 real tokens as 91 full cubes: an odd cube count leaves the
    # second query cube of the last workgroup empty
    Workload("dense-real-tokens-h2", B=1, H=2, T=4, Hh=4, Ww=364, d=128, dtype="bf16", topk=91,
             structure="field", alpha=0.5),
    Workload("dense-ragged-d64", B=2, H=1, T=9, Hh=3, Ww=10, d=64, dtype="bf16", topk=9,
             structure="offset", alpha=0.5),
    Workload("dense-one-token", B=1, H=1, T=1, Hh=1, Ww=1, d=128, dtype="bf16", topk=1,
             structure="offset", alpha=0.5),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_dense_matches_all_cubes_attention(w):
    grid = (w.T, w.Hh, w.Ww)
    x = inputs.make_inputs(w, seed=0)
    t = {n: inputs.as_torch(x[n], w.dtype, DEV) for n in "qkv"}
    cube = {n: vsa.reorder(t[n], grid) for n in "qkv"}
    o, lse = vsa.dense(cube["q"], cube["k"], cube["v"], grid)
    torch.cuda.synchronize()
    g = vo.geometry(w.T, w.Hh, w.Ww)
    qc, kc, vc = (vo.reorder(x[n].astype(np.float64), g) for n in "qkv")
    idx = np.broadcast_to(np.arange(g["C"], dtype=np.int32), (w.B, w.H, g["C"], g["C"]))
    ref_o, ref_lse = vo.fine(qc, kc, vc, idx, g)
    rows = g["valid"]
    assert_close(o.float().cpu().numpy(), ref_o, w.dtype, "O dense", rows=rows)
    assert_close(lse.cpu().numpy()[..., None], ref_lse[..., None], w.dtype, "LSE dense", rows=rows)
    # and the sparse kernel with every cube selected gives the same attention
    of, _ = vsa.fine(cube["q"], cube["k"], cube["v"],
                     torch.from_numpy(idx.copy()).to(DEV), grid)
    assert_close(of.float().cpu().numpy(), ref_o, w.dtype, "O fine, K = C", rows=rows)
