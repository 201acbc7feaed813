"""Pins of the oracle's FP8 (E4M3) functions, independent of the oracle itself.

* The E4M3 value table and round-to-nearest conversion are checked against
  PyTorch's float8_e4m3fn dtype (a library implementation of the same OCP
  format), and ties against the round-half-to-even rule directly.
* The scale exponent is checked against its definition (smallest e with
  amax <= 448 * 2^e) by brute force over e.
* The per-cube quantization is checked against the E4M3 error bound, and
  fine_fp8 against fine on inputs that are already representable.
"""
import numpy as np
import pytest
import torch

from oracle import vsa_oracle as vo

TORCH_TABLE = (torch.arange(256, dtype=torch.int32).to(torch.uint8)
               .view(torch.float8_e4m3fn).double().numpy())
FINITE = np.where(np.isfinite(TORCH_TABLE))[0]


def test_e4m3_decode_matches_library_table():
    mine = vo.e4m3_decode(np.arange(256))
    assert np.array_equal(np.isnan(mine), np.isnan(TORCH_TABLE))
    assert np.array_equal(mine[FINITE], TORCH_TABLE[FINITE])
    assert vo.e4m3_decode(np.array([0x7E]))[0] == 448.0          # largest finite
    assert vo.e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9      # smallest subnormal
    assert vo.e4m3_decode(np.array([0x08]))[0] == 2.0 ** -6      # smallest normal


def test_e4m3_encode_inverts_decode():
    vals = vo.e4m3_decode(FINITE)
    codes = vo.e4m3_encode(vals)
    # +0 and -0 decode to equal values but keep their sign bit
    assert np.array_equal(codes, FINITE.astype(np.uint8))


def test_e4m3_round_matches_library_conversion():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(200_000) * 40, rng.standard_normal(50_000) * 0.02,
                        rng.uniform(-448, 448, 50_000)]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    got = vo.e4m3_round(x.astype(np.float64))
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(got, want)


def test_e4m3_ties_round_to_even():
    pos = np.sort(vo.e4m3_decode(FINITE[(FINITE < 0x7F)]))
    pos = np.unique(pos[pos >= 0])
    mid = (pos[:-1] + pos[1:]) / 2          # exactly halfway: float64 holds it exactly
    out = vo.e4m3_round(mid)
    codes = vo.e4m3_encode(out)
    assert np.all(codes & 1 == 0), "a tie did not round to the even code"
    assert np.all((out == pos[:-1]) | (out == pos[1:]))


def test_e4m3_round_rejects_out_of_range():
    with pytest.raises(ValueError):
        vo.e4m3_round(np.array([470.0]))     # would round to 480, beyond 448
    assert vo.e4m3_round(np.array([463.9]))[0] == 448.0


def test_fp8_scale_exponent_is_the_smallest_fitting_power():
    rng = np.random.default_rng(3)
    amax = np.concatenate([np.exp(rng.uniform(-40, 60, 5000)),
                           448.0 * 2.0 ** np.arange(-20, 20, dtype=np.float64),
                           np.nextafter(448.0 * 2.0 ** np.arange(-20, 20, dtype=np.float64), np.inf),
                           [0.0, 1e-40, 2.0 ** -130, 3.0e38]])
    e = vo.fp8_scale_exponent(amax)
    for a, ei in zip(amax, e):
        # brute force over the exponent range
        cands = [k for k in range(-120, 130) if a <= 448.0 * 2.0 ** k]
        assert ei == cands[0], (a, ei, cands[0])
    assert vo.fp8_scale_exponent(np.array([448.0]))[0] == 0
    assert vo.fp8_scale_exponent(np.array([224.0]))[0] == -1
    assert vo.fp8_scale_exponent(np.array([450.0]))[0] == 1


def _geometry_and_cubes(rng, T=5, Hh=6, Ww=7, d=128, H=2):
    g = vo.geometry(T, Hh, Ww)
    x = rng.standard_normal((1, H, T * Hh * Ww, d))
    return g, vo.reorder(x, g)


def test_quantize_cubes_fp8_error_bound_and_layout():
    rng = np.random.default_rng(11)
    g, xc = _geometry_and_cubes(rng)
    # per-cube magnitudes spread over many binades
    C = g["C"]
    scale = 2.0 ** rng.integers(-30, 30, size=(1, 2, C))
    xc = xc * np.repeat(scale, 64, axis=-1)[..., None]
    codes, e, deq = vo.quantize_cubes_fp8(xc, g)
    assert codes.dtype == np.uint8 and codes.shape == xc.shape and e.shape == (1, 2, C)
    s = np.repeat(np.ldexp(1.0, e), 64, axis=-1)[..., None]
    assert np.array_equal(vo.e4m3_decode(codes) * s, deq)
    y = xc / s                                   # scaled values, |y| <= 448 by the scale rule
    assert np.abs(y).max() <= 448.0
    err = np.abs(deq - xc) / s
    normal = np.abs(y) >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(y[normal]))
    assert np.all(err[~normal] <= 2.0 ** -10)
    # each cube uses the top binade: scaled amax in (224, 448]
    cube_amax = np.abs(y).reshape(1, 2, C, 64 * 128).max(axis=-1)
    assert np.all((cube_amax > 224.0) & (cube_amax <= 448.0))
    pad = ~g["valid"]
    assert np.all(codes[..., pad, :] == 0) and np.all(deq[..., pad, :] == 0)


def test_fine_fp8_equals_fine_on_representable_inputs():
    """Inputs that are E4M3 values times 2^e with cube amax exactly 448 * 2^e
    quantize to themselves, so the FP8 oracle must agree with the exact one."""
    rng = np.random.default_rng(5)
    g = vo.geometry(5, 6, 7)
    C, d, H = g["C"], 128, 2
    vals = vo.e4m3_decode(FINITE)
    out = []
    for _ in range(3):
        codes = rng.choice(vals[np.abs(vals) <= 64], size=(1, H, 64 * C, d))
        e = rng.integers(-8, 8, size=(1, H, C))
        x = codes * np.repeat(np.ldexp(1.0, e), 64, axis=-1)[..., None]
        x[..., ~g["valid"], :] = 0.0
        # plant 448 * 2^e at a valid slot of each cube so that the scale is 2^e
        first = np.array([np.flatnonzero(g["valid"][64 * c: 64 * c + 64])[0] + 64 * c
                          for c in range(C)])
        x[..., first, 0] = 448.0 * np.ldexp(1.0, e)
        out.append(x)
    qc, kc, vc = out
    qc = qc / 64.0   # keep the scores moderate (a power of two: still representable)
    idx = np.stack([np.sort(rng.choice(C, size=3, replace=False)) for _ in range(H * C)])
    idx = idx.reshape(1, H, C, 3)
    o8, lse8, quant = vo.fine_fp8(qc, kc, vc, idx, g)
    o, lse = vo.fine(qc, kc, vc, idx, g)
    rows = g["valid"]
    assert np.array_equal(o8[..., rows, :], o[..., rows, :])
    assert np.array_equal(lse8[..., rows], lse[..., rows])
    for (codes, e), x in zip(quant, (qc, kc, vc)):
        s = np.repeat(np.ldexp(1.0, e), 64, axis=-1)[..., None]
        assert np.array_equal(vo.e4m3_decode(codes) * s, x)
