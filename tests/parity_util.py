"""Shared helpers of the GPU parity tests: tolerances, comparison against the
oracle, structured probe inputs.  Test infrastructure only."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

# O tolerance by input dtype (fp32 accumulate in every case); lse tolerance.
O_TOL = {torch.float32: 1e-5, torch.float16: 1e-2, torch.bfloat16: 1e-2}
LSE_TOL = 1e-3
MANTISSA_BITS = {torch.float16: 10, torch.bfloat16: 7, torch.float32: 23}


def say(*a):
    """Name the case before a GPU step (flushed, so a failing box shows it)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def half_ulp(ref: np.ndarray, dtype) -> np.ndarray:
    """Half a unit in the last place of `dtype` at |ref| (normal range)."""
    mb = MANTISSA_BITS[dtype]
    e = np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -14)))
    return 0.5 * 2.0 ** (e - mb)


def compare(o, lse, o_ref, lse_ref, in_dtype, tag=""):
    """Element-wise gate.  fp32 output: |o - ref| <= O_TOL[in].  Output in the
    input dtype: |o - ref| <= O_TOL[in] + half an ulp of that dtype at ref
    (the rounding of the stored value itself).  lse: <= LSE_TOL.  No NaN or
    Inf anywhere.  Returns (max O error, max lse error)."""
    out_f32 = o.dtype == torch.float32
    o = o.detach().to("cpu").double().numpy()
    lse = lse.detach().to("cpu").double().numpy()
    assert np.isfinite(o).all(), "%s: non-finite O" % tag
    assert np.isfinite(lse).all(), "%s: non-finite lse" % tag
    err = np.abs(o - o_ref)
    lim = O_TOL[in_dtype] if out_f32 else O_TOL[in_dtype] + half_ulp(o_ref, in_dtype)
    bad = err > lim
    assert not bad.any(), "%s: %d O elements over tolerance, max err %.3g" % (
        tag, int(bad.sum()), float(err.max()))
    lerr = np.abs(lse - lse_ref)
    assert lerr.max() <= LSE_TOL, "%s: lse max err %.3g" % (tag, float(lerr.max()))
    return float(err.max()), float(lerr.max())


def position_inputs(N, d, dtype, reverse, B=1, H=1):
    """Position-decoding probe.  K row j holds the binary digits of j (or of
    N-1-j when reverse) in channels 0..nbits-1, V row j the digits of j, Q row
    i holds alpha*2^c in channel c.  Then q_i.k_j = alpha*j (or
    alpha*(N-1-j)) exactly in fp32, consecutive logits differ by
    scale*alpha >= 20, the softmax is one-hot at the largest (smallest)
    visible key and rounding the output recovers that key's index."""
    nbits = max(1, (N - 1).bit_length())
    assert nbits <= d
    j = np.arange(N)
    code = (N - 1 - j) if reverse else j
    bits_k = ((code[:, None] >> np.arange(nbits)[None, :]) & 1).astype(np.float32)
    bits_v = ((j[:, None] >> np.arange(nbits)[None, :]) & 1).astype(np.float32)
    if dtype == torch.float16:
        alpha, scale = 1.0, 24.0          # keeps alpha*2^c below fp16's max
    else:
        alpha, scale = 256.0, 1.0 / math.sqrt(128.0)
    qrow = np.zeros(d, np.float32)
    qrow[:nbits] = alpha * 2.0 ** np.arange(nbits)
    q = np.broadcast_to(qrow, (B, H, N, d)).copy()
    k = np.zeros((B, H, N, d), np.float32)
    v = np.zeros((B, H, N, d), np.float32)
    k[..., :nbits] = bits_k
    v[..., :nbits] = bits_v
    t = lambda x: torch.from_numpy(x).to(dtype)
    return t(q), t(k), t(v), scale, nbits


def decode_positions(o, nbits):
    """Key index encoded in each output row (digits rounded), and the largest
    distance of any digit from 0/1."""
    o = o.detach().to("cpu").double().numpy()
    digits = o[..., :nbits]
    r = np.rint(digits)
    return (r * (2.0 ** np.arange(nbits))).sum(-1).astype(np.int64), float(np.abs(digits - r).max())


def expected_range(N, mask, window):
    i = np.arange(N)
    if mask == "none":
        return np.zeros(N, np.int64), np.full(N, N - 1)
    if mask == "causal":
        return np.zeros(N, np.int64), i
    return np.maximum(0, i - window + 1), i
