"""CPU checks of the seeded input generator (synth/): rounding against library routines,
determinism, and the distributions the workloads ask for."""
from fractions import Fraction

import numpy as np
import torch

import synth


def test_bf16_from_f32_matches_torch_rounding():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-30, 30, 100000))).astype(np.float32)
    want = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.bf16_from_f32(x), want)


def test_f16_from_f32_matches_numpy_rounding():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-25, 12, 100000))).astype(np.float32)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(synth.f16_from_f32(x), want)


def test_bf16_from_f64_rounds_once_to_nearest_even():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(2000) * 4
    # include exact ties between two bf16 neighbours
    base = synth.f32_from_bf16(synth.bf16_from_f32(x.astype(np.float32))).astype(np.float64)
    ulp = np.abs(base) * 2.0 ** -7
    x = np.concatenate([x, base + ulp / 2, base - ulp / 2])
    got = synth.f32_from_bf16(synth.bf16_from_f64(x)).astype(np.float64)
    for xi, gi in zip(x[::7], got[::7]):
        # nearest bf16 by exact rational arithmetic, ties to even significand
        e = int(np.floor(np.log2(abs(xi))))
        step = Fraction(2) ** (e - 7)
        fx = Fraction(xi)
        lo = (fx / step).__floor__() * step
        hi = lo + step
        dl, dh = fx - lo, hi - fx
        if dl < dh:
            want = lo
        elif dh < dl:
            want = hi
        else:
            want = lo if (lo / step) % 2 == 0 else hi
        assert Fraction(gi) == want, (xi, gi, float(want))


def test_generator_is_deterministic_and_keyed():
    a = synth.kv(synth.DT_BF16, 0, synth.T_K, 3, 1, 2, 4, 16, 10, 20)
    b = synth.kv(synth.DT_BF16, 0, synth.T_K, 3, 1, 2, 4, 16, 10, 20)
    np.testing.assert_array_equal(a, b)
    c = synth.kv(synth.DT_BF16, 0, synth.T_K, 3, 1, 2, 4, 16, 15, 10)
    np.testing.assert_array_equal(a[5:15], c)  # position-keyed: windows agree
    d = synth.kv(synth.DT_BF16, 1, synth.T_K, 3, 1, 2, 4, 16, 10, 20)
    assert (a != d).mean() > 0.9


def test_normal_moments_and_range():
    k = synth.stream_key(0, synth.T_K, 0, 0, 0, 0)
    n = synth.normal_f32(k, np.arange(400000, dtype=np.uint64)).astype(np.float64)
    assert abs(n.mean()) < 0.01 and abs(n.var() - 1.0) < 0.01
    assert np.abs(n).max() <= 6.0


def test_ripening_noise_grows_with_the_loop_index():
    """Huginn-shaped planes, the workload's literal formula: plane r - plane R has standard deviation
    0.88^(R-1-r), which grows with r (0.019 at r = 0, 0.88 at r = R - 2)."""
    R = 32
    deep = synth.f32_from_bf16(synth.kv(synth.DT_BF16, 0, synth.T_K, 0, 0, R - 1, 2, 96, 0, 512, synth.MODE_RIPEN,
                                        R)).astype(np.float64)
    for r in (0, 16, 30):
        pr = synth.f32_from_bf16(synth.kv(synth.DT_BF16, 0, synth.T_K, 0, 0, r, 2, 96, 0, 512, synth.MODE_RIPEN,
                                          R)).astype(np.float64)
        sd = (pr - deep).std()
        assert abs(sd / 0.88 ** (R - 1 - r) - 1.0) < 0.05, (r, sd)


def test_ripening_noise_in_the_page_direction_shrinks_with_the_loop_index():
    """MODE_RIPEN_PAPER, the RIPE page's direction (Sec. 3.2: the difference to the deepest plane shrinks
    geometrically as the loop index grows): plane r - plane R has standard deviation 0.88^(r+1) (0.88 at r = 0,
    0.019 at r = R - 2), and the deepest plane is the same as under the workload's recipe."""
    R = 32
    deep = synth.kv(synth.DT_BF16, 0, synth.T_K, 0, 0, R - 1, 2, 96, 0, 512, synth.MODE_RIPEN_PAPER, R)
    assert np.array_equal(deep, synth.kv(synth.DT_BF16, 0, synth.T_K, 0, 0, R - 1, 2, 96, 0, 512, synth.MODE_RIPEN, R))
    deep = synth.f32_from_bf16(deep).astype(np.float64)
    for r in (0, 16, 30):
        pr = synth.f32_from_bf16(synth.kv(synth.DT_BF16, 0, synth.T_K, 0, 0, r, 2, 96, 0, 512,
                                          synth.MODE_RIPEN_PAPER, R)).astype(np.float64)
        sd = (pr - deep).std()
        assert abs(sd / 0.88 ** (r + 1) - 1.0) < 0.05, (r, sd)


def test_codes_and_metadata_ranges():
    c4 = synth.codes(0, synth.T_KCODE, 0, 0, 0, 2, 32, 0, 500, 4)
    c2 = synth.codes(0, synth.T_KCODE, 0, 0, 0, 2, 32, 0, 500, 2)
    assert c4.max() <= 15 and c2.max() <= 3 and abs(c4.mean() - 7.5) < 0.1 and abs(c2.mean() - 1.5) < 0.05
    m = synth.meta(0, 0, 0, 0, 0, 2, 64, 0, 10, 4).view(np.float16).astype(np.float64)
    assert np.all((m[..., 0] >= 0.5) & (m[..., 0] <= 0.75))
    assert np.all((m[..., 1] > -7.0) & (m[..., 1] < -3.0))


def test_cell_plan_draws_and_keeps_final_loop_int4():
    plan = synth.cell_plan(0, 24, 4)
    assert np.all(plan[:, 3] == synth.CELL_INT4)
    frac = [(plan[:, :3] == k).mean() for k in (synth.CELL_INT4, synth.CELL_INT2, synth.CELL_SHARED)]
    big = synth.cell_plan(5, 400, 4)[:, :3]
    frac = [(big == k).mean() for k in (synth.CELL_INT4, synth.CELL_INT2, synth.CELL_SHARED)]
    assert abs(frac[0] - 0.5) < 0.05 and abs(frac[1] - 0.3) < 0.05 and abs(frac[2] - 0.2) < 0.05
