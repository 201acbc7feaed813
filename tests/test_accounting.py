"""Host-side accounting and workload shapes, pinned to the numbers the pages
state (tests/golden/page_facts.json) and to the configuration table."""
import json
import os

import numpy as np
import pytest

from block_sparse_attention_cube_amd import flops
from synth import configs, inputs

FACTS = {f["id"]: f for f in json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                                         "page_facts.json")))["facts"]}


def test_sparsity_gives_the_stated_flop_reduction():
    f = FACTS["sparsity_flops"]
    w = configs.DIT_410M                       # the 410M scaling shape, K = 8 of 64
    assert 1 - w.topk / w.C == f["sparsity"]
    dense = flops.fine_forward_flops(w.B, w.H, w.C, w.C, w.d)
    sparse = flops.fine_forward_flops(w.B, w.H, w.C, w.topk, w.d)
    assert dense == f["attention_flop_reduction"] * sparse
    # same ratio at the Wan-1.3B shape (14 of 112)
    w = configs.WAN_1_3B
    assert flops.fine_forward_flops(1, 12, 112, 112, 128) == 8 * flops.fine_forward_flops(1, 12, 112, 14, 128)


def test_block_is_a_4x4x4_cube():
    assert FACTS["block"]["block_tokens"] == 4 ** 3 == flops.BLOCK


def test_topk_ratio_and_kept_fraction():
    f = FACTS["topk_ratio"]
    k = configs.topk_from_ratio(f["topk_ratio"], configs.WAN_14B.C)
    assert k == configs.WAN_14B.topk == 144
    assert 1 - k / configs.WAN_14B.C == pytest.approx(f["sparsity"])
    g = FACTS["kept_blocks"]
    k3 = configs.topk_from_ratio(g["kept_fraction"], 112)
    assert k3 == 3 and abs(k3 / 112 - g["kept_fraction"]) < 0.5 / 112


def test_workload_table():
    rows = {w.name: (w.N, w.C, w.Np) for w in configs.ALL}
    assert rows["tiny-f32"] == (512, 8, 512)
    assert rows["dit410m"] == (4096, 64, 4096)
    assert rows["wan1.3b-480p"] == (5824, 112, 7168)
    assert rows["wan14b-720p"] == (75600, 1440, 92160)
    # the pages put a 5 s 720P video at over 80k tokens; the workload's 21x45x80
    # grid holds 75,600 real tokens and runs padded to 24x48x80 = 92,160 slots,
    # which is the sequence the kernels process
    assert configs.WAN_14B.Np >= FACTS["wan14b_tokens"]["min_tokens"]
    assert configs.WAN_14B.Np == 92_160 and configs.WAN_14B.N == 75_600
    assert [w.topk for w in configs.SWEEP] == [22, 11, 3]


def test_flop_figures_of_the_survey_table():
    assert flops.fine_forward_flops(1, 12, 112, 14, 128) == 39_460_012_032   # 4*128*64*64*12*112*14
    assert flops.dense_flops(1, 12, 7168, 128) == flops.fine_forward_flops(1, 12, 112, 112, 128)
    assert flops.fine_backward_flops(1, 12, 112, 22, 128) * 2 == 5 * flops.fine_forward_flops(1, 12, 112, 22, 128)


def test_useful_flops_count_valid_pairs_only():
    n = np.array([64, 32, 16])
    idx = np.array([[[[0, 1], [1, 2], [0, 2]]]])
    got = flops.useful_fine_flops(1, 1, 8, n, idx)
    want = 4 * 8 * (64 * (64 + 32) + 32 * (32 + 16) + 16 * (64 + 16))
    assert got == want
    assert got <= flops.fine_forward_flops(1, 1, 3, 2, 8)


def test_generator_is_seeded_and_bf16_exact():
    w = configs.DIT_410M
    a = inputs.make_inputs(w, seed=0, heads=[3])
    b = inputs.make_inputs(w, seed=0, heads=[3])
    c = inputs.make_inputs(w, seed=1, heads=[3])
    assert np.array_equal(a["q"], b["q"]) and not np.array_equal(a["q"], c["q"])
    bits = a["q"].view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)            # bf16 values held in float32
    # per-head streams: generating one head alone equals slicing all heads
    full = inputs.make_inputs(configs.TINY_F32, seed=0)
    one = inputs.make_inputs(configs.TINY_F32, seed=0, heads=[1])
    assert np.array_equal(full["k"][:, 1], one["k"][:, 0])


def test_smooth_field_is_normalised_per_channel():
    w = configs.WAN_1_3B
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([7, 0, 0])))
    f = inputs._field_structure(w, rng).astype(np.float64)
    np.testing.assert_allclose(f.mean(axis=0), 0, atol=1e-5)
    np.testing.assert_allclose(np.sqrt((f * f).mean(axis=0)), 1, atol=1e-5)


def test_sample_plan_covers_the_corner_cube():
    heads, qcubes = inputs.sample_plan(configs.WAN_14B)
    assert len(set(heads)) == 4 and len(qcubes) == 16
    assert 0 in qcubes and configs.WAN_14B.C - 1 in qcubes


def _brute_executed(grid, d, idx):
    """Executed FLOPs by enumeration: every query wave (16 slots: a time
    slice or an h-row) with a valid slot, times every selected key half
    (32 keys: time slices 0-1 or 2-3) with a valid slot, 2 x 16 x 32 x d
    FLOPs each for S and PV."""
    T, Hh, Ww = grid
    ct, ch, cw = -(-T // 4), -(-Hh // 4), -(-Ww // 4)
    cubes = [(t, h, x) for t in range(ct) for h in range(ch) for x in range(cw)]
    rows = flops.query_wave_rows(T, Hh, Ww)
    total = 0
    B, H, C, K = idx.shape
    for b in range(B):
        for hd in range(H):
            for i, (t, h, x) in enumerate(cubes):
                if rows == "t":
                    waves = sum(1 for w in range(4) if 4 * t + w < T)
                else:
                    waves = sum(1 for w in range(4) if 4 * h + w < Hh)
                for k in range(K):
                    tj = cubes[idx[b, hd, i, k]][0]
                    halves = sum(1 for half in range(2) if 4 * tj + 2 * half < T)
                    total += waves * halves * 2 * (2 * 16 * 32 * d)
    return total


def test_wave_rows_follow_the_idle_count():
    # Wan-1.3B: T = 16 leaves no idle time slice, Hh = 14 idles half of the
    # last cube row -> h-rows; Wan-14B: 3 idle time slices per cube column in
    # the last layer (720) against 3 idle h-rows in the last cube row (360)
    assert flops.query_wave_rows(16, 14, 26) == "h"
    assert flops.query_wave_rows(21, 45, 80) == "t"
    assert flops.query_wave_rows(16, 16, 16) == "t"


@pytest.mark.parametrize("grid", [(16, 14, 26), (21, 45, 80), (5, 6, 7), (6, 5, 9), (9, 3, 10)])
def test_executed_flops_match_enumeration(grid):
    rng = np.random.default_rng(sum(grid))
    T, Hh, Ww = grid
    C = -(-T // 4) * -(-Hh // 4) * -(-Ww // 4)
    K = min(C, 5)
    idx = np.stack([rng.permutation(C)[:K] for _ in range(2 * C)]).reshape(1, 2, C, K)
    if C > 200:   # enumeration on a subset of query cubes keeps the test fast
        pick = rng.choice(C, 40, replace=False)
        sub = np.zeros_like(idx)
        sub[..., pick, :] = idx[..., pick, :]
        idx = sub
    assert flops.executed_fine_flops(grid, 64, idx) == _brute_executed(grid, 64, idx)


def test_executed_flops_closed_forms():
    # Wan-1.3B: every cube is four time slices deep (no empty key half); the
    # last of 4 cube rows holds 2 h-rows, so 28 of 112 query cubes run 2 waves
    idx = np.zeros((1, 12, 112, 14), dtype=np.int64)
    got = flops.executed_fine_flops((16, 14, 26), 128, idx)
    assert got * 8 == flops.fine_forward_flops(1, 12, 112, 14, 128) * 7      # (84 + 14) / 112
    # Wan-14B: the last of 6 cube layers (240 of 1440 cubes) is one slice
    # deep: those query cubes run 1 of 4 waves, and as selected cubes they
    # run 1 of 2 halves.  With every selection in the first layer:
    idx = np.zeros((1, 1, 1440, 144), dtype=np.int64)
    full = flops.fine_forward_flops(1, 1, 1440, 144, 128)
    assert flops.executed_fine_flops((21, 45, 80), 128, idx) * 8 == full * 7  # (1200 + 60) / 1440
    # ... and every selection in the last layer: half of that
    idx[:] = 1439
    assert flops.executed_fine_flops((21, 45, 80), 128, idx) * 16 == full * 7
