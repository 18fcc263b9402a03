"""The seeded input generator (seeded_inputs.py): determinism, the pinned
bytes of every workload, and the round-to-nearest-even casts it relies on.

The generator holds no attention arithmetic; these tests pin what both the
oracle and the GPU path read.  The casts are checked against an independent
definition of nearest-even rounding onto the target grid, computed exactly in
float64 (a float32 value and a power-of-two spacing need no rounding there).
"""
import math
import os

import numpy as np
import pytest
import torch

import seeded_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "input_sha256.txt")


def _golden():
    rows = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, hq, hk, hv = line.split()
        rows[name] = (hq, hk, hv)
    return rows


def test_draws_are_deterministic_and_depend_on_the_seed():
    a = si.make_qkv(2, 3, 17, 8, "bf16", 1234)
    b = si.make_qkv(2, 3, 17, 8, "bf16", 1234)
    c = si.make_qkv(2, 3, 17, 8, "bf16", 1235)
    for x, y, z in zip(a, b, c):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
        assert not torch.equal(x.view(torch.int16), z.view(torch.int16))
    # q, k and v are three different draws of one stream, in that order
    assert not torch.equal(a[0], a[1]) and not torch.equal(a[1], a[2])
    rng = np.random.default_rng(1234)
    first = rng.standard_normal((2, 3, 17, 8), dtype=np.float32)
    second = rng.standard_normal((2, 3, 17, 8), dtype=np.float32)
    assert torch.equal(a[0], torch.from_numpy(first).to(torch.bfloat16))
    assert torch.equal(a[1], torch.from_numpy(second).to(torch.bfloat16))


def test_shared_and_dout_variants_follow_the_same_stream():
    q, k, v = si.make_qkv(1, 4, 9, 8, "f16", 77)
    q2, k2, v2 = si.make_qkv_shared(1, 4, 4, 9, 8, "f16", 77)
    q3, k3, v3, do = si.make_qkv_dout(1, 4, 9, 8, "f16", 77)
    for x, y, z in ((q, q2, q3), (k, k2, k3), (v, v2, v3)):
        assert torch.equal(x, y) and torch.equal(x, z)
    assert do.shape == q.shape and not torch.equal(do, q)


@pytest.mark.parametrize("name", sorted(_golden()))
def test_workload_bytes_match_the_pinned_hashes(name):
    w = si.BY_NAME[name]
    q, k, v = si.make_workload(w)
    assert tuple(q.shape) == (w.B, w.H, w.N, w.d)
    assert tuple(k.shape) == (w.B, w.kv_heads, w.N, w.d)
    assert (si.sha256(q), si.sha256(k), si.sha256(v)) == _golden()[name]


def test_every_configured_workload_is_pinned():
    pinned = set(_golden())
    assert {w.name for w in si.WORKLOADS} <= pinned
    assert {w.name for w in si.FP8_WORKLOADS} <= pinned


def _nearest_even(x32: np.ndarray, mant_bits: int, emin: int) -> np.ndarray:
    """Round float32 values to the grid of a binary format with `mant_bits`
    stored mantissa bits and smallest normal exponent `emin` (subnormals
    below it), nearest value, ties to the even neighbour.  Exact in float64.
    Overflow is not handled (the inputs stay far inside both ranges)."""
    x = x32.astype(np.float64)
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    # log2 of a float64 can be off by one at binade edges: correct it exactly
    e = np.where(np.exp2(e) > ax, e - 1, e)
    e = np.where(np.exp2(e + 1) <= ax, e + 1, e)
    e = np.maximum(e, emin)
    spacing = np.exp2(e - mant_bits)
    n = np.floor(ax / spacing)
    lo = n * spacing
    rem = ax - lo
    half = spacing / 2
    up = (rem > half) | ((rem == half) & (np.mod(n, 2) == 1))
    r = np.where(up, lo + spacing, lo)
    return np.where(x < 0, -r, r)


@pytest.mark.parametrize("dtype,mant,emin", [("bf16", 7, -126), ("f16", 10, -14)])
def test_cast_is_round_to_nearest_even(dtype, mant, emin):
    rng = np.random.default_rng(5)
    x = rng.standard_normal(200_000, dtype=np.float32)
    # add exact halfway points between neighbours of the target grid (ties)
    # and values one float32 ulp either side of them
    base = np.array([1.0, 1.5, 3.0, 0.7, -2.25, 5.5e-5, -1e-6, 3e-7], dtype=np.float64)
    e = np.floor(np.log2(np.abs(base)))
    sp = np.exp2(np.maximum(e, emin) - mant)
    ties = (np.floor(np.abs(base) / sp) + 0.5) * sp * np.sign(base)
    ties = np.concatenate([ties, ties + sp, -ties])
    t32 = ties.astype(np.float32)
    assert np.all(t32.astype(np.float64) == ties)  # the ties are exact float32 values
    near = np.concatenate([np.nextafter(t32, np.float32(np.inf)), np.nextafter(t32, np.float32(-np.inf))])
    allx = np.concatenate([x, t32, near])
    want = _nearest_even(allx, mant, emin)
    got = torch.from_numpy(allx).to(si.DTYPES[dtype]).to(torch.float64).numpy()
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:10]
    # the generator's own output is this cast of its float32 draws
    rng = np.random.default_rng(1002)
    draw = rng.standard_normal((1, 2, 64, 16), dtype=np.float32)
    q = si.make_qkv(1, 2, 64, 16, dtype, 1002)[0]
    assert np.array_equal(q.to(torch.float64).numpy().ravel(), _nearest_even(draw.ravel(), mant, emin))


def test_nearest_even_reference_on_hand_cases():
    """The reference rounding itself, on cases worked by hand: bf16 keeps 8
    significant bits, so 1 + 2^-8 is halfway between 1 and 1 + 2^-7 and goes
    to the even one (1); 1 + 3 * 2^-8 is halfway between 1 + 2^-7 and
    1 + 2^-6 and goes to 1 + 2^-6; f16 keeps 11 bits."""
    f = np.float32
    cases = [(1 + 2 ** -8, 7, 1.0), (1 + 3 * 2 ** -8, 7, 1 + 2 ** -6), (1 + 2 ** -9, 7, 1.0),
             (1 + 2 ** -8 + 2 ** -20, 7, 1 + 2 ** -7), (-(1 + 2 ** -8), 7, -1.0),
             (1 + 2 ** -11, 10, 1.0), (1 + 3 * 2 ** -11, 10, 1 + 2 ** -9), (2.0 ** -25, 10, 0.0),
             (3 * 2.0 ** -25, 10, 2.0 ** -23)]
    for x, mant, want in cases:
        emin = -126 if mant == 7 else -14
        got = _nearest_even(np.array([x], dtype=f), mant, emin)[0]
        assert got == want, (x, got, want)
    assert math.isclose(_nearest_even(np.array([0.1], dtype=f), 7, -126)[0], 0.10009765625)
