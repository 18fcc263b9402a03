"""Pins for the 8-bit parts of the oracle (decode_e4m3, attention_fp8,
attention_weights_rows): each is checked against something other than
itself.

The pages name FP8 for the Hopper version ("FlashAttention (NL)", section
"FlashAttention-3 (2024)") without fixing a format; the format is OCP E4M3,
the one gfx950's 8-bit matrix instructions read.  Pins:
  * torch's float8_e4m3fn -> float64 conversion of all 256 codes (library);
  * closed forms of the format: 1.0, the largest finite value 448, the
    smallest subnormal 2^-9 and normal 2^-6, NaN only at S.1111.111, the
    sign bit, equal spacing across the subnormal/normal boundary, each
    binade twice the one below, strictly increasing codes;
  * torch's round-to-nearest cast lands on the nearest decoded value;
  * attention_fp8 on a case worked by hand, and its V-factor linearity;
  * attention_weights_rows against the C oracle's o and lse (an independent
    route to the same softmax);
  * planted mistakes in a private copy of decode_e4m3 are caught.
"""
import inspect
import math

import numpy as np
import pytest
import torch

import oracle

ALL = np.arange(256, dtype=np.uint8)


def torch_values():
    return torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).double().numpy()


# ---- pins, each taking the decoder under test --------------------------------
def pin_matches_torch(dec):
    np.testing.assert_array_equal(dec(ALL), torch_values())


def pin_closed_forms(dec):
    v = dec(ALL)
    assert v[0x38] == 1.0 and v[0x40] == 2.0 and v[0x30] == 0.5
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and math.copysign(1.0, v[0x80]) == -1.0
    nan = np.isnan(v)
    assert nan[0x7F] and nan[0xFF] and nan.sum() == 2


def pin_structure(dec):
    v = dec(ALL)
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must increase strictly"
    # the subnormal spacing continues into the first normal binade
    np.testing.assert_array_equal(np.diff(v[:17]), np.full(16, 2.0 ** -9))
    # every normal binade doubles the one below
    for c in range(8, 0x7F - 8):
        assert v[c + 8] == 2 * v[c], hex(c)
    np.testing.assert_array_equal(v[0x80:0xFF], -v[:0x7F])


def pin_torch_cast_is_nearest(dec):
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 100,
                        rng.standard_normal(2000) * 1e-3]).astype(np.float32)
    codes = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = dec(codes)
    table = dec(ALL[:0x7F])
    nearest = np.abs(np.abs(x.astype(np.float64))[:, None] - table[None, :]).min(axis=1)
    np.testing.assert_array_equal(np.abs(np.abs(x) - np.abs(got)), nearest)
    assert np.all((np.sign(got) == np.sign(x)) | (got == 0))


PINS = [pin_matches_torch, pin_closed_forms, pin_structure, pin_torch_cast_is_nearest]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_decode_pins(pin):
    pin(oracle.decode_e4m3)


def test_decode_accepts_torch_tensors():
    t = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn)
    np.testing.assert_array_equal(oracle.decode_e4m3(t), torch_values())
    np.testing.assert_array_equal(oracle.decode_e4m3(t.view(torch.uint8)), torch_values())
    with pytest.raises(ValueError):
        oracle.decode_e4m3([0, 256])


# ---- attention on decoded inputs ---------------------------------------------
def codes(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)


def test_attention_fp8_hand_case():
    # q = [1], [1]; k = [1], [0]; v = [2], [-1]; scale 0.5, V factor 3
    q = codes([[[[1.0], [1.0]]]])
    k = codes([[[[1.0], [0.0]]]])
    v = codes([[[[2.0], [-1.0]]]])
    e = math.exp(0.5)
    o, lse = oracle.attention_fp8(q, k, v, 0.5, 3.0, "causal")
    np.testing.assert_allclose(o[0, 0, :, 0], [6.0, 3.0 * (2 * e - 1) / (e + 1)], rtol=1e-15)
    np.testing.assert_allclose(lse[0, 0], [0.5, math.log(e + 1)], rtol=1e-15)
    o, lse = oracle.attention_fp8(q, k, v, 0.5, 3.0, "none")
    np.testing.assert_allclose(o[0, 0, :, 0], [3.0 * (2 * e - 1) / (e + 1)] * 2, rtol=1e-15)


def test_attention_fp8_v_factor_and_shared_heads():
    rng = np.random.default_rng(9)
    q = codes(rng.standard_normal((1, 4, 30, 16)))
    k = codes(rng.standard_normal((1, 2, 30, 16)))
    v = codes(rng.standard_normal((1, 2, 30, 16)))
    o1, l1 = oracle.attention_fp8(q, k, v, 0.25, 1.0, "sliding", 7)
    o2, l2 = oracle.attention_fp8(q, k, v, 0.25, -2.5, "sliding", 7)
    np.testing.assert_array_equal(o2, -2.5 * o1)
    np.testing.assert_array_equal(l1, l2)
    # heads 0, 1 read key/value head 0; heads 2, 3 head 1
    oh, lh = oracle.attention_fp8(q[:, 3:4], k[:, 1:2], v[:, 1:2], 0.25, 1.0, "sliding", 7)
    np.testing.assert_array_equal(oh[0, 0], o1[0, 3])
    np.testing.assert_array_equal(lh[0, 0], l1[0, 3])


def test_attention_fp8_refuses_nan_codes():
    q = torch.full((1, 1, 2, 4), 0x7F, dtype=torch.uint8)
    k = torch.zeros((1, 1, 2, 4), dtype=torch.uint8)
    with pytest.raises(ValueError):
        oracle.attention_fp8(q, k, k, 1.0)


@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("sliding", 5)])
def test_weights_rows_agree_with_the_c_oracle(mask, window):
    rng = np.random.default_rng(12)
    N, d = 70, 12
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    pos = np.array([0, 1, 4, 33, 69])
    W = oracle.attention_weights_rows(q[pos], pos, k, 0.3, mask, window)
    o, lse = oracle.attention_rows(q[pos], pos, k, v, 0.3, mask, window)
    np.testing.assert_allclose(W @ v, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(W.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    s = 0.3 * q[pos] @ k.T
    for r, i in enumerate(pos):
        vis = np.array([oracle.visible(int(i), j, mask, window) for j in range(N)])
        assert np.all(W[r, ~vis] == 0.0)
        np.testing.assert_allclose(W[r, vis], np.exp(s[r, vis] - lse[r]), rtol=1e-13)


# ---- planted mistakes -----------------------------------------------------------
SRC = inspect.getsource(oracle.decode_e4m3)
MUTANTS = {
    "bias_8": ("np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    "subnormal_scale": ("m * 2.0 ** -9", "m * 2.0 ** -10"),
    "mantissa_16ths": ("(1.0 + m / 8.0)", "(1.0 + m / 16.0)"),
    "no_implicit_one": ("(1.0 + m / 8.0)", "(m / 8.0)"),
    "nan_at_m6": ("(e == 15) & (m == 7)", "(e == 15) & (m == 6)"),
    "no_nan": ("np.where((e == 15) & (m == 7), np.nan, mag)", "mag"),
    "sign_ignored": ("np.where(sign == 1, -mag, mag)", "mag"),
    "exponent_3_bits": ("e = (c >> 3) & 15", "e = (c >> 3) & 7"),
}


def mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, "mutation site not unique: %s" % name
    ns = {"np": np, "_codes": oracle._codes}
    exec(SRC.replace(old, new), ns)
    return ns["decode_e4m3"]


def failing_pins(dec):
    failed = []
    for pin in PINS:
        try:
            pin(dec)
        except Exception:
            failed.append(pin.__name__)
    return failed


def test_unmodified_copy_passes_every_pin():
    ns = {"np": np, "_codes": oracle._codes}
    exec(SRC, ns)
    assert failing_pins(ns["decode_e4m3"]) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_decode_mutant_is_caught(name):
    assert failing_pins(mutant(name)), "mutant %s passed every pin" % name
