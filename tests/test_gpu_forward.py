"""GPU parity of the forward path (reorder, coarse, fine, whole forward) against
the fp64 oracle, through the C ABI (ctypes binding)."""
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
    Workload("ragged-bf16-d128", B=2, H=3, T=5, Hh=6, Ww=7, d=128, dtype="bf16", topk=3,
             structure="offset", alpha=0.5),
    Workload("ragged-f32-d128", B=1, H=2, T=6, Hh=5, Ww=9, d=128, dtype="f32", topk=4,
             structure="offset", alpha=1.0),
    Workload("ragged-bf16-d64", B=1, H=2, T=9, Hh=3, Ww=10, d=64, dtype="bf16", topk=2,
             structure="field", alpha=0.5),
    Workload("ragged-f32-d64", B=2, H=1, T=3, Hh=7, Ww=5, d=64, dtype="f32", topk=2,
             structure="field", alpha=0.5),
    # last cube layer two time slices deep: its query waves 2, 3 hold only pads
    # and its key cubes take the half-depth V staging and score tiles
    Workload("ragged-t2-bf16-d128", B=1, H=2, T=6, Hh=5, Ww=9, d=128, dtype="bf16", topk=4,
             structure="offset", alpha=0.5),
    Workload("one-token", B=1, H=2, T=1, Hh=1, Ww=1, d=128, dtype="bf16", topk=1,
             structure="offset", alpha=0.5),
    Workload("all-cubes", B=1, H=2, T=8, Hh=12, Ww=10, d=128, dtype="bf16", topk=18,
             structure="field", alpha=0.5),
    Workload("one-cube-each", B=1, H=2, T=8, Hh=12, Ww=10, d=64, dtype="bf16", topk=1,
             structure="field", alpha=0.5),
    # the top-K holds ceil(C/64) keys per lane, rounded up to a power of two:
    # 288 cubes take the 8-key form, 640 cubes the 16-key form (ragged edges)
    Workload("cubes288-ragged", B=1, H=2, T=15, Hh=31, Ww=36, d=64, dtype="bf16", topk=16,
             structure="field", alpha=0.5),
    Workload("cubes640-ragged", B=1, H=2, T=16, Hh=62, Ww=39, d=128, dtype="bf16", topk=20,
             structure="field", alpha=0.5),
    # 2304 cubes: above 2048 the coarse stage takes 8 query cubes per workgroup
    # and the top-K 64 keys per lane
    Workload("cubes2304-ragged", B=1, H=1, T=4, Hh=190, Ww=189, d=64, dtype="bf16", topk=3,
             structure="offset", alpha=0.5),
    # one-frame last cube layer (its key cubes' empty second halves skipped)
    # with more than 64 selected cubes per query cube (the per-lane key
    # table reloads mid-walk)
    Workload("t13-k70", B=1, H=1, T=13, Hh=16, Ww=24, d=64, dtype="bf16", topk=70,
             structure="field", alpha=0.5),
]
SMALL = [configs.TINY_F32, configs.DIT_410M, configs.WAN_1_3B]
CASES = SMALL + EDGE
ids = lambda ws: [w.name for w in ws]


def dev(x, w):
    return inputs.as_torch(x, w.dtype, DEV)


def host(t):
    return t.float().cpu().numpy()


def grid(w):
    return (w.T, w.Hh, w.Ww)


@pytest.fixture(scope="module")
def cache():
    return {}


def case_data(w, cache):
    """Inputs, GPU cube-order copies and the oracle forward, computed once per workload."""
    if w.name not in cache:
        x = inputs.make_inputs(w, seed=0)
        q, k, v = (dev(x[n], w) for n in "qkv")
        cube = tuple(vsa.reorder(t, grid(w)) for t in (q, k, v))
        ref = vo.forward(x["q"], x["k"], x["v"], w.T, w.Hh, w.Ww, w.topk)
        cache[w.name] = (x, (q, k, v), cube, ref)
    return cache[w.name]


@pytest.mark.parametrize("w", CASES, ids=ids(CASES))
def test_reorder_is_bit_exact(w, cache):
    x, (q, _, _), (qc, _, _), ref = case_data(w, cache)
    g = ref["geometry"]
    got = host(qc)
    np.testing.assert_array_equal(got, vo.reorder(x["q"], g))
    back = vsa.reorder(qc, grid(w), inverse=True)
    assert torch.equal(back, q)


@pytest.mark.parametrize("w", CASES, ids=ids(CASES))
def test_coarse_scores_selection_and_output(w, cache):
    x, _, (qc, kc, vc), ref = case_data(w, cache)
    oc, idx, sc = vsa.coarse(qc, kc, vc, grid(w), w.topk, return_scores=True)
    torch.cuda.synchronize()
    sc = sc.cpu().numpy().astype(np.float64)
    scale = max(1.0, float(np.abs(ref["scores"]).max()))
    np.testing.assert_allclose(sc, ref["scores"], rtol=0, atol=2e-5 * scale)
    check_idx(idx.cpu().numpy(), ref["idx"], ref["scores"], w.topk)
    assert_close(host(oc), ref["oc"], w.dtype, "O_coarse per cube")


@pytest.mark.parametrize("w", CASES, ids=ids(CASES))
def test_fine_with_oracle_selection(w, cache):
    x, _, (qc, kc, vc), ref = case_data(w, cache)
    g = ref["geometry"]
    idx = torch.from_numpy(ref["idx"]).to(DEV)
    o, lse = vsa.fine(qc, kc, vc, idx, grid(w))
    torch.cuda.synchronize()
    assert_close(host(o), ref["o_fine_cube"], w.dtype, "O_fine (oracle idx)", rows=g["valid"])
    assert_close(lse.cpu().numpy()[..., None], ref["lse_cube"][..., None], w.dtype, "LSE",
                 rows=g["valid"])


@pytest.mark.parametrize("w", CASES, ids=ids(CASES))
def test_fine_selection_order_does_not_matter(w, cache):
    x, _, (qc, kc, vc), ref = case_data(w, cache)
    g = ref["geometry"]
    rng = np.random.default_rng(3)
    perm = np.array([[[rng.permutation(r) for r in hh] for hh in bb] for bb in ref["idx"]])
    o, _ = vsa.fine(qc, kc, vc, torch.from_numpy(perm.astype(np.int32)).to(DEV), grid(w))
    assert_close(host(o), ref["o_fine_cube"], w.dtype, "O_fine (permuted idx)", rows=g["valid"])


@pytest.mark.parametrize("w", CASES, ids=ids(CASES))
def test_forward_end_to_end(w, cache):
    x, (q, k, v), _, ref = case_data(w, cache)
    o_fine, o_coarse, idx, lse = vsa.forward(q, k, v, grid(w), w.topk)
    torch.cuda.synchronize()
    gidx = idx.cpu().numpy()
    near = check_idx(gidx, ref["idx"], ref["scores"], w.topk)
    # check the fine stage on the mask the GPU chose (identical unless near ties)
    ref_g = ref if near == 0 else vo.forward(x["q"], x["k"], x["v"], w.T, w.Hh, w.Ww, w.topk,
                                             idx=gidx)
    assert_close(host(o_fine), ref_g["o_fine"], w.dtype, "O_fine raster")
    assert_close(host(o_coarse), ref["o_coarse"], w.dtype, "O_coarse raster")
    g = ref["geometry"]
    assert_close(lse.cpu().numpy()[..., None], ref_g["lse_cube"][..., None], w.dtype, "LSE",
                 rows=g["valid"])


@pytest.mark.parametrize("w", [configs.WAN_1_3B, EDGE[0]], ids=ids([configs.WAN_1_3B, EDGE[0]]))
def test_forward_is_deterministic(w, cache):
    _, (q, k, v), _, _ = case_data(w, cache)
    a = [t.clone() for t in vsa.forward(q, k, v, grid(w), w.topk)]
    b = vsa.forward(q, k, v, grid(w), w.topk)
    for s, t in zip(a, b):
        assert torch.equal(s, t)


def _forward_sampled(w):
    """vsa_forward at full size on the GPU against the oracle on sampled heads
    (whole coarse stage) and sampled query cubes of each."""
    x = inputs.make_inputs(w, seed=0)
    q, k, v = (dev(x[n], w) for n in "qkv")
    o_fine, o_coarse, idx, lse = vsa.forward(q, k, v, grid(w), w.topk)
    torch.cuda.synchronize()
    heads, qcubes = inputs.sample_plan(w)
    hs = torch.tensor(heads, device=DEV)
    sub = {n: x[n][:, heads] for n in "qkv"}
    del x
    gidx = idx[:, hs].cpu().numpy()
    ref = vo.forward(sub["q"], sub["k"], sub["v"], w.T, w.Hh, w.Ww, w.topk, qcubes=qcubes,
                     idx=None)
    check_idx(gidx, ref["idx"], ref["scores"], w.topk)
    ref_g = vo.forward(sub["q"], sub["k"], sub["v"], w.T, w.Hh, w.Ww, w.topk, qcubes=qcubes,
                       idx=gidx)
    g = ref_g["geometry"]
    pos = np.concatenate([np.arange(64 * c, 64 * c + 64) for c in qcubes])
    pos = pos[g["valid"][pos]]
    toks = g["token"][pos]
    assert_close(host(o_fine[:, hs])[:, :, toks], ref_g["o_fine"][:, :, toks], w.dtype,
                 "O_fine sampled")
    assert_close(host(o_coarse[:, hs]), ref["o_coarse"], w.dtype, "O_coarse sampled heads")
    assert_close(lse[:, hs].cpu().numpy()[..., pos, None], ref_g["lse_cube"][..., pos, None],
                 w.dtype, "LSE sampled")


def test_forward_one_coarse_workgroup_per_row_tile():
    """384 row tiles of 16 query cubes (16 per head x 24 heads): above the CU
    count, so one coarse workgroup per row tile computes O_coarse and the
    top-K from one copy of the scores (the small shapes split them)."""
    w = Workload("coarse-fused", B=1, H=24, T=16, Hh=32, Ww=32, d=64, dtype="bf16", topk=24,
                 structure="field", alpha=0.5)
    _forward_sampled(w)


def test_forward_wan14b_sampled():
    """Wan-14B 720p shape at full size on the GPU; the oracle checks 4 sampled
    heads (full coarse stage) and 16 query cubes of each of them."""
    w = configs.WAN_14B
    x = inputs.make_inputs(w, seed=0)
    q, k, v = (dev(x[n], w) for n in "qkv")
    o_fine, o_coarse, idx, lse = vsa.forward(q, k, v, grid(w), w.topk)
    torch.cuda.synchronize()
    heads, qcubes = inputs.sample_plan(w)
    hs = torch.tensor(heads, device=DEV)
    sub = {n: x[n][:, heads] for n in "qkv"}
    del x
    gidx = idx[:, hs].cpu().numpy()
    ref = vo.forward(sub["q"], sub["k"], sub["v"], w.T, w.Hh, w.Ww, w.topk, qcubes=qcubes,
                     idx=None)
    check_idx(gidx, ref["idx"], ref["scores"], w.topk)
    ref_g = vo.forward(sub["q"], sub["k"], sub["v"], w.T, w.Hh, w.Ww, w.topk, qcubes=qcubes,
                       idx=gidx)
    g = ref_g["geometry"]
    pos = np.concatenate([np.arange(64 * c, 64 * c + 64) for c in qcubes])
    pos = pos[g["valid"][pos]]
    toks = g["token"][pos]
    assert_close(host(o_fine[:, hs])[:, :, toks], ref_g["o_fine"][:, :, toks], w.dtype,
                 "O_fine sampled")
    assert_close(host(o_coarse[:, hs]), ref["o_coarse"], w.dtype, "O_coarse sampled heads")
    assert_close(lse[:, hs].cpu().numpy()[..., pos, None], ref_g["lse_cube"][..., pos, None],
                 w.dtype, "LSE sampled")


@pytest.mark.parametrize("w", CASES, ids=ids(CASES))
def test_fine_raster_is_the_forward_fine_stage(w, cache):
    """vsa_fine_raster on the forward's own selection gives the forward's
    O_fine bit for bit (same kernel) and, with the per-cube coarse rows,
    O_coarse broadcast to every valid token; fp32 problems are refused."""
    x, (q, k, v), (qc, kc, vc), ref = case_data(w, cache)
    o_fine, o_coarse, idx, lse = vsa.forward(q, k, v, grid(w), w.topk)
    oc, _ = vsa.coarse(qc, kc, vc, grid(w), w.topk)
    if w.dtype == "f32":
        with pytest.raises(vsa.VSAError):
            vsa.fine_raster(q, k, v, idx, grid(w), oc=oc)
        return
    of, lse2, ocr = vsa.fine_raster(q, k, v, idx, grid(w), oc=oc)
    torch.cuda.synchronize()
    assert torch.equal(of, o_fine)
    g = ref["geometry"]
    valid = torch.from_numpy(g["valid"]).to(DEV)
    assert torch.equal(lse2[..., valid], lse[..., valid])
    assert_close(host(ocr), ref["o_coarse"], w.dtype, "O_coarse broadcast")
    of_only, _, none = vsa.fine_raster(q, k, v, idx, grid(w), return_lse=False)
    assert none is None and torch.equal(of_only, o_fine)
