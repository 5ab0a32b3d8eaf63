"""The MXFP8 oracle against its pins, and planted mistakes that the pins must catch (CPU only)."""
import numpy as np
import pytest

import oracle.mxfp8 as M
import oracle_mx_pins as P


@pytest.mark.parametrize("pin", P.ALL_MX_PINS, ids=lambda f: f.__name__)
def test_mx_pin(pin):
    pin(M)


def _fails(pin):
    try:
        pin(M)
    except AssertionError:
        return True
    return False


def test_planted_scale_rounded_up(monkeypatch):
    """ceil instead of floor in the shared exponent (one of the published variants, not the spec's)."""
    def bad(amax):
        amax = np.asarray(amax, np.float64)
        se = np.where(amax > 0, np.ceil(np.log2(np.where(amax > 0, amax, 1.0))) - 8, -127)
        return np.clip(se, -127, 127).astype(np.int64)
    monkeypatch.setattr(M, "shared_exponent", bad)
    assert _fails(P.pin_mx_scale_rule)


def test_planted_emax_off_by_one(monkeypatch):
    monkeypatch.setattr(M, "E4M3_EMAX", 7)
    assert _fails(P.pin_mx_scale_rule)


def test_planted_ties_away_from_zero(monkeypatch):
    pos = M.e4m3_values()[:0x7F]           # codes 0 .. 0x7E, ascending

    def bad(a):
        a = np.asarray(a, np.float64)
        mag = np.minimum(np.abs(a), 448.0)
        hi = np.clip(np.searchsorted(pos, mag), 0, pos.size - 1)
        lo = np.clip(hi - 1, 0, pos.size - 1)
        pick = np.where(pos[hi] - mag <= mag - pos[lo], hi, lo)
        return ((np.signbit(a).astype(np.int64) << 7) | pick).astype(np.uint8)
    monkeypatch.setattr(M, "e4m3_encode", bad)
    assert _fails(P.pin_e4m3_encode_matches_torch) and _fails(P.pin_e4m3_ties_and_saturation)


def test_planted_no_saturation(monkeypatch):
    """Values above 448 X wrap to NaN (the non-saturating cast) instead of 448."""
    real = M.e4m3_encode
    monkeypatch.setattr(M, "e4m3_encode", lambda a: np.where(np.abs(np.asarray(a)) > 448, np.uint8(0x7F), real(a)))
    assert _fails(P.pin_mx_scale_rule)


def test_planted_scale_on_wrong_block(monkeypatch):
    """Scales applied to the wrong blocks (reversed order)."""
    real = M.dequantize
    monkeypatch.setattr(M, "dequantize", lambda c, s: real(c, np.asarray(s)[..., ::-1]))
    assert _fails(P.pin_mx_dot_is_block_factored) and _fails(P.pin_mx_round_trip_bound)


def test_planted_weights_quantised_along_n(monkeypatch):
    """Weight blocks along the output columns instead of along K."""
    real = M.fake_quant

    def bad(v, axis=-1):
        v = np.asarray(v)
        return real(v, axis=1 if (v.ndim == 2 and axis == 0) else axis)
    monkeypatch.setattr(M, "fake_quant", bad)
    assert _fails(P.pin_mx_layer_identical_experts_is_quantised_mlp)


def test_planted_h_not_quantised(monkeypatch):
    real = M.fake_quant
    calls = []

    def bad(v, axis=-1):
        calls.append(axis)
        if axis == 1 and len(calls) > 1:          # the h quantisation inside expert_ffn
            return np.asarray(v, np.float64)
        return real(v, axis)
    monkeypatch.setattr(M, "fake_quant", bad)
    assert _fails(P.pin_mx_layer_identical_experts_is_quantised_mlp)
