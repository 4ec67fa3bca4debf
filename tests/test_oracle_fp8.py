"""CPU pins of the FP8 oracle: E4M3 code points fixed by the format's
definition, an integer-arithmetic construction of every code's value, the
round trip with the input encoder (an independent implementation),
a pure-Python brute force of the descaled, transposed-V attention, and
planted mistakes these pins must catch."""
import math
import os
import types

import numpy as np
import pytest

from fa_inputs import f32_to_e4m3, make_fp8
from oracle import decode_e4m3, reference_attention, reference_attention_fp8

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

# (code, value) fixed by the E4M3 definition: bias 7, 3 mantissa bits,
# subnormals m 2^-9, S.1111.111 NaN, largest finite 448
CODE_POINTS = [(0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
               (0x08, 2.0 ** -6), (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875),
               (0x40, 2.0), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0),
               (0x81, -(2.0 ** -9))]


def pin_code_points(dec):
    for c, want in CODE_POINTS:
        assert dec(np.array([c]))[0] == want, hex(c)
    assert np.isnan(dec(np.array([0x7F]))[0]) and np.isnan(dec(np.array([0xFF]))[0])
    assert math.copysign(1.0, dec(np.array([0x80]))[0]) == -1.0


def pin_every_code_by_integers(dec):
    """value(c) = (8 + m) 2^(e - 10) for e >= 1, m 2^-9 for e = 0, with the
    sign bit on top, built with integer powers only."""
    from fractions import Fraction
    got = dec(np.arange(256))
    for c in range(256):
        e, m = (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            assert np.isnan(got[c])
            continue
        mag = Fraction(m, 512) if e == 0 else Fraction(8 + m) * Fraction(2) ** (e - 10)
        want = -mag if c & 0x80 else mag
        assert Fraction(float(got[c])) == want, hex(c)


def pin_round_trip_with_encoder(dec):
    c = np.arange(256)
    v = dec(c)
    fin = np.isfinite(v)
    assert np.array_equal(f32_to_e4m3(v[fin]), c[fin].astype(np.uint8))


def _brute(q8, k8, vt8, qd, kd, vd, causal, scale, dec):
    """Pure-Python loops: decode each element, scale it, attend."""
    B, Hq, Nq, d = q8.shape
    Hkv, Nk = k8.shape[1], k8.shape[2]
    qd, kd, vd = (np.asarray(x, dtype=np.float64) for x in (qd, kd, vd))
    O = np.zeros((B, Hq, Nq, d))
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(Nq):
                keys = [j for j in range(Nk) if not causal or j <= i + Nk - Nq]
                s = [scale * sum(float(dec(np.array([q8[b, h, i, t]]))[0]) * qd[b, h] *
                                 float(dec(np.array([k8[b, g, j, t]]))[0]) * kd[b, g]
                                 for t in range(d)) for j in keys]
                if not s:
                    continue
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                z = sum(w)
                for t in range(d):
                    O[b, h, i, t] = sum(wj * float(dec(np.array([vt8[b, g, t, j]]))[0]) * vd[b, g]
                                        for wj, j in zip(w, keys)) / z
    return O


def pin_brute_force_descaled_transposed(attn_and_dec):
    attn, dec = attn_and_dec
    q8, k8, vt8, qd, kd, vd = make_fp8(2, 4, 2, 3, 5, 3, seed=9)
    for causal in (False, True):
        O, _ = attn(q8, k8, vt8, qd, kd, vd, causal=causal, scale=0.4)
        Ob = _brute(q8, k8, vt8, qd, kd, vd, causal, 0.4, dec)
        np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)


def _decoder_pins():
    return [pin_code_points, pin_every_code_by_integers,
            pin_round_trip_with_encoder]


@pytest.mark.parametrize("pin", _decoder_pins(), ids=lambda p: p.__name__)
def test_decoder_pins(pin):
    pin(decode_e4m3)


def test_fp8_attention_brute_force():
    pin_brute_force_descaled_transposed((reference_attention_fp8, decode_e4m3))


def test_fp8_attention_is_the_definition_on_decoded_inputs():
    """With power-of-two descales the decoded inputs are exact bf16-range
    numbers: the result is the plain forward oracle on them."""
    q8, k8, vt8, _, _, _ = make_fp8(1, 2, 1, 6, 9, 4, seed=10)
    qd = np.full((1, 2), 0.25, np.float32)
    kd = np.full((1, 1), 0.5, np.float32)
    vd = np.full((1, 1), 2.0, np.float32)
    O, lse = reference_attention_fp8(q8, k8, vt8, qd, kd, vd, causal=True,
                                     scale=0.3)
    q = decode_e4m3(q8) * 0.25
    k = decode_e4m3(k8) * 0.5
    v = (decode_e4m3(vt8) * 2.0).transpose(0, 1, 3, 2)
    O2, l2 = reference_attention(q, k, v, causal=True, scale=0.3)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(lse, l2)


def test_make_fp8_uses_full_range_per_head():
    q8, k8, vt8, qd, kd, vd = make_fp8(2, 4, 2, 64, 80, 16, seed=11)
    for x8 in (q8, k8, vt8):
        mags = np.abs(decode_e4m3(x8)).reshape(x8.shape[0], x8.shape[1], -1)
        assert np.all(mags.max(axis=2) == 448.0)
    assert qd.shape == (2, 4) and kd.shape == (2, 2) and vd.shape == (2, 2)


_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "oracle", "fp8.py")
MUTANTS = {
    "bias_off_by_one": ("2.0 ** (e - 7)", "2.0 ** (e - 8)"),
    "sign_ignored": ("sign = np.where(c & 0x80, -1.0, 1.0)", "sign = 1.0"),
    "subnormal_scale": ("m * 2.0 ** -9", "m * 2.0 ** -10"),
    "v_not_transposed": ("v = vt.transpose(0, 1, 3, 2)", "v = vt"),
    "descale_q_for_k": ("k = decode_e4m3(k8) * np.asarray(k_descale",
                        "k = decode_e4m3(k8) * np.asarray(v_descale"),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_fp8_pins_catch_planted_mistake(name):
    old, new = MUTANTS[name]
    src = open(_SRC).read()
    assert src.count(old) == 1, old
    src = src.replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType("fp8_mutant")
    exec(compile(src.replace(old, new), "fp8_mutant", "exec"), mod.__dict__)
    failed = []
    for pin in _decoder_pins():
        try:
            pin(mod.decode_e4m3)
        except Exception:
            failed.append(pin.__name__)
    try:
        pin_brute_force_descaled_transposed((mod.reference_attention_fp8,
                                             decode_e4m3))
    except Exception:
        failed.append("brute")
    assert failed, name
