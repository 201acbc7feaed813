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


def test_executed_flops_skip_query_waves_past_the_t_extent():
    # Wan-1.3B: T = 16, every cube four time slices deep -> all block FLOPs run
    w = configs.WAN_1_3B
    nt = [min(4, w.T - 4 * t) for t in range(-(-w.T // 4)) for _ in range(w.C // (-(-w.T // 4)))]
    assert flops.executed_fine_flops(1, 12, 14, 128, nt) == flops.fine_forward_flops(1, 12, 112, 14, 128)
    # Wan-14B: T = 21, the last of 6 cube layers holds one time slice -> 1 of 4 waves
    w = configs.WAN_14B
    layers = -(-w.T // 4)
    per_layer = w.C // layers
    nt = [min(4, w.T - 4 * t) for t in range(layers) for _ in range(per_layer)]
    assert nt.count(1) == 240
    got = flops.executed_fine_flops(1, 40, 144, 128, nt)
    full = flops.fine_forward_flops(1, 40, 1440, 144, 128)
    assert got * 8 == full * 7          # (1200 + 240/4) / 1440 = 7/8
    # brute force over cubes and waves
    brute = sum(4 * 128 * 16 * 64 * 144 * 40 for c in range(w.C) for wave in range(4) if wave < nt[c])
    assert got == brute
