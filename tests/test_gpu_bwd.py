"""GPU parity of the backward pass (fa_bwd) against the fp64 oracle
(oracle.attention_bwd / _rows / _keys).

* whole tensors over both 16-bit types, both head dims, the three masks
  and ragged N (one to several tiles, with a tail);
* the long-context shape at full size (B=1 H=32 N=16384 d=128, causal), in
  the launch configuration the benchmark times: sampled query rows (dq)
  and keys (dk, dv) against the oracle one by one;
* logits four times larger; a window of one key (dv = dout exactly);
  determinism; errors reported before any launch.
Tolerance, per tensor: max |g - g_ref| <= 4 u max |g_ref| + 1e-5, u the unit
roundoff of the input type (2^-8 bf16, 2^-11 fp16): every term of a
gradient has one factor (P or dS) rounded to the input type, the output is
rounded once more, and D uses o as stored in the input type.
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
    g = got.detach().cpu().double().numpy() if hasattr(got, "detach") else got
    assert np.isfinite(g).all(), "%s: non-finite values" % tag
    err = np.abs(g - ref).max() if g.size else 0.0
    tol = 4 * UNIT[dtype] * (np.abs(ref).max() if ref.size else 0.0) + 1e-5
    assert err <= tol, "%s: max |err| %.3e > tol %.3e" % (tag, err, tol)


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
        rq, rk, rv = oracle.attention_bwd(q, k, v, do, scale, mask, window)
        for nm, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            check(g, r, dtype, "%s N=%d" % (nm, N))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_bwd_large_logits(dtype):
    for mult in (4.0,):
        q, k, v, do = si.make_qkv_dout(1, 3, 700, 128, dtype, 9300)
        q = (q.float() * mult).to(si.DTYPES[dtype])
        for mask, window in (("none", 0), ("causal", 0), ("sliding", 77)):
            say("bwd stress", dtype, mult, mask)
            scale = 1.0 / math.sqrt(128)
            dq, dk, dv = grads(q, k, v, do, scale, mask, window)
            rq, rk, rv = oracle.attention_bwd(q, k, v, do, scale, mask, window)
            for nm, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
                check(g, r, dtype, "%s x%g %s" % (nm, mult, mask))


def test_bwd_full_size_sampled():
    """B=1 H=32 N=16384 d=128 bf16 causal (the benchmark's shape and
    launch): sampled rows and keys of two heads against the oracle."""
    B, H, N, d = 1, 32, 16384, 128
    say("bwd full size")
    q, k, v, do = si.make_qkv_dout(B, H, N, d, "bf16", 9400)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = grads(q, k, v, do, scale, "causal", 0)
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    rng = np.random.default_rng(9401)
    sel = np.array(sorted(set([0, 1, 63, 64, 127, 128, 8191, N - 2, N - 1]
                              + rng.integers(0, N, size=40).tolist())), dtype=np.int64)
    idx = torch.from_numpy(sel).to(DEV)
    for h in (0, H - 1):
        say("bwd full size head", h)
        rq = oracle.attention_bwd_rows(q[0, h], k[0, h], v[0, h], do[0, h], sel, scale, "causal")
        rk, rv = oracle.attention_bwd_keys(q[0, h], k[0, h], v[0, h], do[0, h], sel, scale, "causal")
        check(dq[0, h].index_select(0, idx), rq, "bf16", "dq h%d" % h)
        check(dk[0, h].index_select(0, idx), rk, "bf16", "dk h%d" % h)
        check(dv[0, h].index_select(0, idx), rv, "bf16", "dv h%d" % h)


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
        rq, rk, rv = oracle.attention_bwd_gqa(q, k, v, do, scale, mask, window)
        for nm, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            check(g, r, dtype, "%s H=%d H_kv=%d N=%d" % (nm, H, H_kv, N))


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
        rq, rk, rv = oracle.attention_bwd_gqa(q, k, v, do, scale, mask, window)
        for nm, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            check(g, r, dtype, "%s B=%d H=%d H_kv=%d N=%d" % (nm, B, H, H_kv, N))


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


def test_bwd_shared_heads_full_size_sampled():
    """B=1 H=32 H_kv=8 N=16384 d=128 bf16 causal: sampled query rows (dq) of
    two query heads and sampled keys (dk, dv summed over the four query
    heads) of the first key/value head against the oracle."""
    B, H, H_kv, N, d = 1, 32, 8, 16384, 128
    g = H // H_kv
    say("bwd shared heads full size")
    q, k, v, do = si.make_qkv_dout_shared(B, H, H_kv, N, d, "bf16", 9900)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = grads(q, k, v, do, scale, "causal", 0)
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    rng = np.random.default_rng(9901)
    sel = np.array(sorted(set([0, 1, 127, 128, 8191, N - 1] + rng.integers(0, N, size=20).tolist())),
                   dtype=np.int64)
    idx = torch.from_numpy(sel).to(DEV)
    for h in (0, g - 1):
        say("bwd shared heads full size dq head", h)
        rq = oracle.attention_bwd_rows(q[0, h], k[0, 0], v[0, 0], do[0, h], sel, scale, "causal")
        check(dq[0, h].index_select(0, idx), rq, "bf16", "dq h%d" % h)
    rk = np.zeros((len(sel), d))
    rv = np.zeros((len(sel), d))
    for h in range(g):
        say("bwd shared heads full size keys, query head", h)
        a, b = oracle.attention_bwd_keys(q[0, h], k[0, 0], v[0, 0], do[0, h], sel, scale, "causal")
        rk += a
        rv += b
    check(dk[0, 0].index_select(0, idx), rk, "bf16", "dk kv0")
    check(dv[0, 0].index_select(0, idx), rv, "bf16", "dv kv0")
