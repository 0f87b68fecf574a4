"""Pins of the oracle's window-exit codec (LoopKV page, Sec. 3.1: KIVI-style codes with an fp16 scale and
zero per group of 32, keys per channel and values per token; Sec. 3.3: INT4 value codes split into hi and lo
bit planes) against facts that do not come from the codec itself: numpy's IEEE half conversion, groups whose
codes are known in closed form, the rounding rule, and the quantisation error bound."""
import numpy as np
import pytest

import oracle


@pytest.mark.filterwarnings("ignore:overflow encountered in cast")
def test_f16_conversion_matches_numpy_ieee_half():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-9, 6, 20000),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, 6.1035156e-05, 5.9604645e-08, 2.9802322e-08,
                  2.9802326e-08, 8.940697e-08, 1.0009765625, 1.00048828125, 1.00146484375, 2049.0, 2051.0,
                  np.inf, -np.inf], dtype=np.float32)])
    for x in vals:
        want = int(np.array([x], dtype=np.float32).astype(np.float16).view(np.uint16)[0])
        assert oracle.f16_from_f32(float(x)) == want, x
    for h in range(0, 0x10000):
        if (h & 0x7C00) == 0x7C00 and (h & 0x3FF):
            continue  # NaN payloads
        want = float(np.array([h], dtype=np.uint16).view(np.float16).astype(np.float32)[0])
        assert oracle.f32_from_f16(h) == want


def _f16(x):
    return int(np.array([x], dtype=np.float32).astype(np.float16).view(np.uint16)[0])


@pytest.mark.parametrize("bits", [4, 2])
def test_exact_grid_round_trips(bits):
    """A group lying exactly on a grid z + sigma c (z, sigma exact in fp16, every value exact in fp32) whose
    extremes are codes 0 and 2^b - 1 is encoded to exactly those codes and that metadata."""
    levels = (1 << bits) - 1
    sigma, z = 0.375, -2.5
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, levels + 1, (32, 64)).astype(np.uint8)
    codes[0, :] = 0
    codes[1, :] = levels
    k = (z + sigma * codes).astype(np.float32)
    vcodes = rng.integers(0, levels + 1, (32, 64)).astype(np.uint8)
    vcodes[:, 0] = 0
    vcodes[:, 32] = 0
    vcodes[:, 31] = levels
    vcodes[:, 63] = levels
    v = (z + sigma * vcodes).astype(np.float32)
    kc, km, vc, vm = oracle.kivi_encode(k, v, bits)
    np.testing.assert_array_equal(kc, codes)
    np.testing.assert_array_equal(vc, vcodes)
    assert (km[:, 0] == _f16(sigma)).all() and (km[:, 1] == _f16(z)).all()
    assert (vm[..., 0] == _f16(sigma)).all() and (vm[..., 1] == _f16(z)).all()


def test_constant_group_has_zero_scale_and_zero_codes():
    k = np.full((32, 32), 1.2345, dtype=np.float32)
    v = np.full((32, 32), -7.0, dtype=np.float32)
    kc, km, vc, vm = oracle.kivi_encode(k, v, 4)
    assert not kc.any() and not vc.any()
    assert (km[:, 0] == 0).all() and (km[:, 1] == _f16(1.2345)).all()
    assert (vm[..., 0] == 0).all() and (vm[..., 1] == _f16(-7.0)).all()


def test_half_steps_round_to_even_codes():
    """With mn = 0 and mx = 15 the scale is exactly 1; values at c + 0.5 round to the even neighbour."""
    col = np.array([0.0, 15.0] + [c + 0.5 for c in range(14)] + [3.0] * 16, dtype=np.float32)
    k = np.tile(col[:, None], (1, 32))
    v = np.zeros((32, 32), dtype=np.float32)
    kc, km, _, _ = oracle.kivi_encode(k, v, 4)
    want = [0, 15] + [c + (c % 2) for c in range(14)] + [3] * 16
    np.testing.assert_array_equal(kc[:, 0], want)
    assert km[0, 0] == _f16(1.0) and km[0, 1] == 0


@pytest.mark.parametrize("bits", [4, 2])
def test_error_bound_and_monotonicity(bits):
    """Decoded values z16 + s16 c are within s16 / 2 of x wherever x - z16 lies in the codable range
    [-s16/2, (2^b - 1/2) s16] (up to fp32 rounding of the two operations); codes never decrease as x grows; the
    group's smallest value gets code 0 or 1 and its largest 2^b - 1 or 2^b - 2 (fp16 rounding of the metadata
    moves the grid by less than one step)."""
    levels = (1 << bits) - 1
    rng = np.random.default_rng(10 + bits)
    for trial in range(40):
        scale = 10.0 ** rng.uniform(-3, 2)
        k = (rng.standard_normal((32, 64)) * scale + rng.uniform(-5, 5) * scale).astype(np.float32)
        v = (rng.standard_normal((32, 64)) * scale).astype(np.float32)
        kc, km, vc, vm = oracle.kivi_encode(k, v, bits)
        for ch in range(64):
            s = oracle.f32_from_f16(km[ch, 0])
            z = oracle.f32_from_f16(km[ch, 1])
            x = k[:, ch].astype(np.float64)
            c = kc[:, ch].astype(np.float64)
            inside = (x - z >= -0.5 * s) & (x - z <= (levels + 0.5) * s)
            err = np.abs(x - (z + s * c))
            assert np.all(err[inside] <= 0.5 * s * (1 + 1e-5) + 1e-6 * abs(z))
            order = np.argsort(x, kind="stable")
            assert np.all(np.diff(c[order]) >= 0)
            assert c[np.argmin(x)] in (0, 1) and c[np.argmax(x)] in (levels, levels - 1)
        for t in range(32):
            for g in range(2):
                s = oracle.f32_from_f16(vm[t, g, 0])
                z = oracle.f32_from_f16(vm[t, g, 1])
                x = v[t, 32 * g:32 * g + 32].astype(np.float64)
                c = vc[t, 32 * g:32 * g + 32].astype(np.float64)
                inside = (x - z >= -0.5 * s) & (x - z <= (levels + 0.5) * s)
                assert np.all(np.abs(x - (z + s * c))[inside] <= 0.5 * s * (1 + 1e-5) + 1e-6 * abs(z))


def test_partial_page_uses_only_its_tokens():
    """A page with n < 32 valid tokens takes its key statistics over those tokens only."""
    rng = np.random.default_rng(3)
    k = rng.standard_normal((20, 32)).astype(np.float32)
    v = rng.standard_normal((20, 32)).astype(np.float32)
    kc, km, vc, vm = oracle.kivi_encode(k, v, 4)
    for ch in range(32):
        assert km[ch, 1] == _f16(k[:, ch].min())
        assert km[ch, 0] == _f16(np.float32(k[:, ch].max() - k[:, ch].min()) / np.float32(15.0))
