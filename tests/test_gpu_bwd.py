"""GPU parity of the backward pass (fa_bwd, fa_bwd_gqa) against the fp64
oracle.

* whole tensors over both 16-bit types, both head dims, the three masks
  and ragged N (one to several tiles, with a tail), plain and shared
  key/value heads (with and without the split of a group's query heads);
* the long-context shapes at full size (B=1 H=32 N=16384 d=128, causal, with
  32, 8 and 1 key/value heads), in the launch configuration the benchmark
  times: sampled query rows (dq) and keys (dk, dv) of every head;
* logits four times larger; a window of one key (dv = dout exactly);
  determinism; errors reported before any launch.

Tolerance, per element, from the kernels' rounding steps (u the unit
roundoff of the input type: 2^-8 bf16, 2^-11 fp16).  The kernels recompute
P in fp32, round P (for dv) and dS = P (dP - D) (for dq, dk) to the input
type once per term, accumulate in fp32 and round each gradient once; D_i =
<do_i, o_i> uses o as stored (the forward's error plus one rounding: at most
2u Dm_i, Dm_i = sum_c |do_ic| max_j |v_jc|).  Rounding errors of different
terms are independent and of either sign, so they add in quadrature; four
times the root-sum-square of u x term is about seven standard deviations of
nearest rounding (uniform, variance u^2/3).  With the oracle's sums
(oracle.attention_bwd_terms; rq = scale sqrt(sum_j dS_ij^2 k_jc^2), cq =
scale |sum_j P_ij k_jc|, rk, ck, rv likewise, n* the term counts for fp16's
subnormal steps s, a* the sums of magnitudes):
  |dq - ref| <= 4u rq + 2u Dm cq + 4s nq + u |ref| + g aq + 1e-7
  |dk - ref| <= 4u rk + 2u ck    + 4s nk + u |ref| + g ak + 1e-7
  |dv - ref| <= 4u rv            + 4s nv + u |ref| + g av + 1e-7
g = 4 sqrt(n) 2^-24 + 1e-5 covers fp32 accumulation over the n summed terms
and the recomputed P; u |ref| is the final rounding, 2u Dm cq the error of
D (one value per row, so it enters linearly).  Comparisons of two kernel
results (shared heads against copied heads) keep a per-tensor bound,
4u max |ref| + 1e-5.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_04_amd as fa
import oracle
import seeded_inputs as si
from tests.parity_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
UNIT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()
    yield


def grads(q, k, v, do, scale, mask, window):
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.attention(qd, kd, vd, scale, mask, window)
    dq, dk, dv = fa.attention_bwd(qd, kd, vd, o, lse, dod, scale, mask, window)
    torch.cuda.synchronize()
    return dq, dk, dv


def check(got, ref, dtype, tag):
    """Per-tensor bound, for two kernel results (shared against copied heads)."""
    g = got.detach().cpu().double().numpy() if hasattr(got, "detach") else got
    assert np.isfinite(g).all(), "%s: non-finite values" % tag
    err = np.abs(g - ref).max() if g.size else 0.0
    tol = 4 * UNIT[dtype] * (np.abs(ref).max() if ref.size else 0.0) + 1e-5
    assert err <= tol, "%s: max |err| %.3e > tol %.3e" % (tag, err, tol)


SUBNORMAL_HALF_STEP = {"bf16": 2.0 ** -134, "f16": 2.0 ** -25}


def reference(q, k, v, do, scale, mask, window, rows=None, keys=None, dtype="bf16"):
    """Oracle gradients and per-element tolerances for [B, H, N, d] q, do and
    [B, H_kv, N, d] k, v: dq at `rows` of every query head, dk and dv at
    `keys` of every key/value head (default: all positions).  Terms of a key
    shared by several query heads add (sums) or add in quadrature (root-sum-
    squares)."""
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    grp = H // H_kv
    u, sm = UNIT[dtype], SUBNORMAL_HALF_STEP[dtype]
    o, lse = oracle.attention_gqa(q, k, v, scale, mask, window)
    R = N if rows is None else len(rows)
    K = N if keys is None else len(keys)
    ref = {"dq": np.zeros((B, H, R, d)), "tq": np.zeros((B, H, R, d))}
    acc = {n: np.zeros((B, H_kv, K, d)) for n in ("dk", "dv", "ak", "av", "rk2", "rv2", "ck2",
                                                   "nk2", "nv2")}
    gq = 4 * math.sqrt(N) * 2.0 ** -24 + 1e-5
    for b in range(B):
        for h in range(H):
            hk = oracle.kv_head(h, H, H_kv)
            t = oracle.attention_bwd_terms(q[b, h], k[b, hk], v[b, hk], do[b, h], o[b, h],
                                           lse[b, h], scale, mask, window, rows, keys)
            ref["dq"][b, h] = t["dq"]
            ref["tq"][b, h] = (4 * u * t["rq"] + 2 * u * t["dm"][:, None] * t["cq"]
                               + 4 * sm * t["nq"] + u * np.abs(t["dq"]) + gq * t["aq"] + 1e-7)
            for n in ("dk", "dv", "ak", "av"):
                acc[n][b, hk] += t[n]
            for n in ("rk", "rv", "ck", "nk", "nv"):
                acc[n + "2"][b, hk] += t[n] ** 2
    gk = 4 * math.sqrt(grp * N) * 2.0 ** -24 + 1e-5
    ref["dk"], ref["dv"] = acc["dk"], acc["dv"]
    ref["tk"] = (4 * u * np.sqrt(acc["rk2"]) + 2 * u * np.sqrt(acc["ck2"])
                 + 4 * sm * np.sqrt(acc["nk2"]) + u * np.abs(acc["dk"]) + gk * acc["ak"] + 1e-7)
    ref["tv"] = (4 * u * np.sqrt(acc["rv2"]) + 4 * sm * np.sqrt(acc["nv2"])
                 + u * np.abs(acc["dv"]) + gk * acc["av"] + 1e-7)
    return ref


def check_elem(got, ref, tol, tag):
    """Element-wise gate |got - ref| <= tol; returns the largest err / tol."""
    g = got.detach().cpu().double().numpy() if hasattr(got, "detach") else got
    assert np.isfinite(g).all(), "%s: non-finite values" % tag
    if not g.size:
        return 0.0
    err = np.abs(g - ref)
    bad = err > tol
    assert not bad.any(), "%s: %d of %d elements over tolerance, worst err %.3e (tol %.3e)" % (
        tag, int(bad.sum()), g.size, float(err[bad].max()), float(tol[bad][np.argmax(err[bad])]))
    return float((err / tol).max())


def check_all(dq, dk, dv, ref, tag, rows=None, keys=None):
    """dq (at rows), dk and dv (at keys) against reference(); prints the
    worst error-to-tolerance ratio of each."""
    sel = lambda t, ix: t if ix is None else t.index_select(2, torch.from_numpy(ix).to(t.device))
    rq = check_elem(sel(dq, rows), ref["dq"], ref["tq"], "dq " + tag)
    rk = check_elem(sel(dk, keys), ref["dk"], ref["tk"], "dk " + tag)
    rv = check_elem(sel(dv, keys), ref["dv"], ref["tv"], "dv " + tag)
    say("%s: worst err/tol dq %.2f dk %.2f dv %.2f" % (tag, rq, rk, rv))


RAGGED_N = [1, 2, 31, 63, 64, 65, 127, 128, 129, 200, 257, 1000]
MASKS = [("none", 0), ("causal", 0), ("sliding", 1), ("sliding", 33), ("sliding", 100)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask,window", MASKS)
def test_bwd_ragged_sizes(dtype, d, mask, window):
    for N in RAGGED_N:
        say("bwd ragged", dtype, d, mask, window, N)
        q, k, v, do = si.make_qkv_dout(2, 2, N, d, dtype, 9100 + N + d)
        scale = 1.0 / math.sqrt(d)
        dq, dk, dv = grads(q, k, v, do, scale, mask, window)
        check_all(dq, dk, dv, reference(q, k, v, do, scale, mask, window, dtype=dtype),
                  "N=%d" % N)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_bwd_large_logits(dtype):
    for mult in (4.0,):
        q, k, v, do = si.make_qkv_dout(1, 3, 700, 128, dtype, 9300)
        q = (q.float() * mult).to(si.DTYPES[dtype])
        for mask, window in (("none", 0), ("causal", 0), ("sliding", 77)):
            say("bwd stress", dtype, mult, mask)
            scale = 1.0 / math.sqrt(128)
            dq, dk, dv = grads(q, k, v, do, scale, mask, window)
            check_all(dq, dk, dv, reference(q, k, v, do, scale, mask, window, dtype=dtype),
                      "x%g %s" % (mult, mask))


def full_size_sel(N, seed, extra=40):
    rng = np.random.default_rng(seed)
    return np.array(sorted(set([0, 1, 63, 64, 127, 128, 255, 256, 8191, N - 2, N - 1]
                               + rng.integers(0, N, size=extra).tolist())), dtype=np.int64)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("H_kv,seed", [(32, 9400), (8, 9900), (1, 9950)],
                         ids=["plain", "gqa8", "mqa"])
def test_bwd_full_size_sampled(H_kv, seed):
    """B=1 H=32 N=16384 d=128 bf16 causal with 32, 8 and 1 key/value heads
    (the benchmark's shapes and launches; with one key/value head the dk/dv
    pass splits each key tile's 32 query heads over 8 workgroups): sampled
    query rows (dq) of every query head and sampled keys (dk, dv, summed over
    the query heads that share them) of every key/value head, against the
    oracle element by element.  (The oracle's forward over the whole tensor
    takes ~20 s on 16 host cores.)"""
    B, H, N, d = 1, 32, 16384, 128
    say("bwd full size", H_kv, "gpu")
    q, k, v, do = si.make_qkv_dout_shared(B, H, H_kv, N, d, "bf16", seed)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = grads(q, k, v, do, scale, "causal", 0)
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    sel = full_size_sel(N, seed + 1)
    say("bwd full size", H_kv, "oracle")
    ref = reference(q, k, v, do, scale, "causal", 0, rows=sel, keys=sel)
    check_all(dq, dk, dv, ref, "full size H_kv=%d" % H_kv, rows=sel, keys=sel)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_bwd_window_of_one_key(dtype):
    # o_i = v_i: dv = dout exactly, dq = dk = 0 up to the fp32 difference
    # between the two evaluations of <dout_i, v_i>
    q, k, v, do = si.make_qkv_dout(1, 2, 1111, 64, dtype, 9500)
    dq, dk, dv = grads(q, k, v, do, 0.125, "sliding", 1)
    assert torch.equal(dv.cpu(), do)
    assert dq.abs().max().item() <= 1e-5 and dk.abs().max().item() <= 1e-5


def test_bwd_is_deterministic():
    q, k, v, do = si.make_qkv_dout(2, 2, 1000, 128, "bf16", 9600)
    a = grads(q, k, v, do, 0.09, "causal", 0)
    b = grads(q, k, v, do, 0.09, "causal", 0)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_errors_before_launch():
    x = torch.zeros(1, 1, 64, 64, dtype=torch.float32, device=DEV)
    lse = torch.zeros(1, 1, 64, dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FaError) as e:
        fa.attention_bwd(x, x, x, x, lse, x)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    y = torch.zeros(1, 1, 64, 256, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fa.FaError) as e:
        fa.attention_bwd(y, y, y, y, lse, y)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    z = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fa.FaError) as e:
        fa.attention_bwd(z, z, z, z, lse, z, mask="sliding", window=0)
    assert e.value.status == fa.FA_ERR_INVALID_ARG


# ---- shared key/value heads (fa_bwd_gqa) --------------------------------------
HEADS = [(4, 1), (4, 2), (6, 3)]  # (H, H_kv)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("sliding", 100)])
def test_bwd_shared_heads_against_oracle(dtype, d, mask, window):
    for (H, H_kv), N in zip(HEADS, [1, 257, 1000]):
        say("bwd shared heads", dtype, d, mask, window, H, H_kv, N)
        q, k, v, do = si.make_qkv_dout_shared(2, H, H_kv, N, d, dtype, 9700 + N + d + H_kv)
        scale = 1.0 / math.sqrt(d)
        dq, dk, dv = grads(q, k, v, do, scale, mask, window)
        assert dk.shape == k.shape and dv.shape == v.shape
        check_all(dq, dk, dv, reference(q, k, v, do, scale, mask, window, dtype=dtype),
                  "H=%d H_kv=%d N=%d" % (H, H_kv, N))


@pytest.mark.parametrize("H,H_kv", [(8, 1), (8, 2)])
def test_bwd_shared_heads_match_copied_heads(H, H_kv):
    """dq equals the plain backward pass on key/value heads copied out to
    every query head bit for bit (same kernel arithmetic); dk, dv equal the
    copies' gradients summed over each group up to rounding (the shared pass
    sums in fp32 and rounds once, the copies round per head)."""
    N, d = 600, 128
    q, k, v, do = si.make_qkv_dout_shared(1, H, H_kv, N, d, "bf16", 9800 + H_kv)
    g = H // H_kv
    kc, vc = (t.repeat_interleave(g, dim=1).contiguous() for t in (k, v))
    for mask, window in (("causal", 0), ("sliding", 50)):
        say("bwd copied heads", H, H_kv, mask)
        dq, dk, dv = grads(q, k, v, do, 0.1, mask, window)
        cq, ck, cv = grads(q, kc, vc, do, 0.1, mask, window)
        assert torch.equal(dq, cq), mask
        sk = ck.float().reshape(1, H_kv, g, N, d).sum(dim=2).double().cpu().numpy()
        sv = cv.float().reshape(1, H_kv, g, N, d).sum(dim=2).double().cpu().numpy()
        check(dk, sk, "bf16", "dk vs copies %s" % mask)
        check(dv, sv, "bf16", "dv vs copies %s" % mask)


# Groups of 8 or more query heads per key/value head with few key tiles: the
# dk/dv pass splits each tile's query heads over kv_parts workgroups (at most
# g / 4) and sums their fp32 partials.  (B, H, H_kv, N): parts 8 (g = 32,
# N = 1000), 2 uneven (g = 9: heads 0-3 and 4-8), 2 (g = 8 with two
# key/value heads), 3 (g = 12), 4 with two batch entries (g = 16).
SPLIT_HEADS = [(1, 32, 1, 1000), (1, 9, 1, 333), (1, 16, 2, 700), (1, 12, 1, 129), (2, 16, 1, 300)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("sliding", 100)])
def test_bwd_split_query_heads_against_oracle(dtype, d, mask, window):
    for B, H, H_kv, N in SPLIT_HEADS:
        say("bwd split query heads", dtype, d, mask, window, B, H, H_kv, N)
        q, k, v, do = si.make_qkv_dout_shared(B, H, H_kv, N, d, dtype, 9750 + N + d + H)
        scale = 1.0 / math.sqrt(d)
        dq, dk, dv = grads(q, k, v, do, scale, mask, window)
        check_all(dq, dk, dv, reference(q, k, v, do, scale, mask, window, dtype=dtype),
                  "B=%d H=%d H_kv=%d N=%d" % (B, H, H_kv, N))


def test_bwd_multi_query_full_size_matches_copied_heads():
    """B=1 H=32 H_kv=1 N=16384 d=128 bf16 causal, the benchmarked multi-query
    shape (dk/dv split over 8 workgroups per key tile): dq equals the plain
    pass on the key/value head copied to all 32 query heads bit for bit; dk,
    dv equal the copies' gradients summed over the heads up to rounding."""
    B, H, H_kv, N, d = 1, 32, 1, 16384, 128
    say("bwd multi-query full size vs copied heads")
    q, k, v, do = si.make_qkv_dout_shared(B, H, H_kv, N, d, "bf16", 9950)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = grads(q, k, v, do, scale, "causal", 0)
    kc, vc = (t.repeat_interleave(H, dim=1).contiguous() for t in (k, v))
    cq, ck, cv = grads(q, kc, vc, do, scale, "causal", 0)
    assert torch.equal(dq, cq)
    sk = ck.float().sum(dim=1, keepdim=True).double().cpu().numpy()
    sv = cv.float().sum(dim=1, keepdim=True).double().cpu().numpy()
    check(dk, sk, "bf16", "dk vs copies")
    check(dv, sv, "bf16", "dv vs copies")
