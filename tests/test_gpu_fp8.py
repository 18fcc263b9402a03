"""GPU parity of the 8-bit forward pass (fa_fwd_fp8) against the oracle
(oracle.attention_fp8: exact fp64 attention of the values the E4M3 codes
stand for, times the V factor).

Tolerance.  The pages give none for FP8 ("FlashAttention (NL)", section
"FlashAttention-3 (2024)", only names the precision), so it is derived from
the kernel's arithmetic, per output element (row i, column c), from the
oracle's fp64 softmax weights W_ij of that row:
  * each probability is rounded to E4M3 before the product with V (scaled
    by 2^3 relative to a reference <= the row maximum): weight error at most
    2^-4 W_ij (3-bit mantissa, nearest even) or, in the subnormal range, 2^-13
    max_j W_ij;
  * the 8-bit matrix instruction sums its 64 products to about 2^-12 of the
    largest of them (measured on gfx950; 2^-11 is used): the score error
    e_i <= scale 2^-11 sum over the two 64-element slices of max |q_ic| max
    |k_jc|, which moves each weight by at most a factor e^(2 e_i), and the
    P V sums lose at most 2^-11 of sum_j W_ij |v_jc| (plus fp32 rounding);
so |o_ic - ref_ic| <= |v_scale| sum_j (max(2^-4 W_ij, 2^-13 max W_i) +
(2.2 e_i + 2^-10.9) W_ij) |v_jc| + 1e-6, plus half an ulp when o is stored in
16 bits; |lse_i - ref_i| <= e_i + 1e-5.  This bound is worst case; because
nearest rounding errors are spread over +-half an ulp, the mean squared O
error must also stay within 4x the mean of sum_j (max(2^-4 W_ij, 2^-13
max W_i))^2 v_jc^2 / 3, which a wrong key or column mapping exceeds by
orders of magnitude.  Inputs whose scores are small integers with
scale = ln 2 make every probability a power of two that E4M3 holds exactly:
there only the product-summation terms remain, a sharp check of the data
paths.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_04_amd as fa
import oracle
import seeded_inputs as si
from tests.parity_util import half_ulp, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LN2_F32 = float(np.float32(math.log(2.0)))
OUT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()
    yield


def run(q8, k8, v8, scale, v_scale=1.0, mask="none", window=0, out="bf16"):
    o, lse = fa.attention_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), scale, v_scale, mask, window,
                              OUT[out])
    torch.cuda.synchronize()
    return o, lse


def slice_bounds(qd, pos, kd, vd, scale, mask, window, v_scale, sharp):
    """Reference rows and their bounds for query rows qd [R, d] at positions
    pos against one key/value slice kd, vd [N, d] (decoded values)."""
    o_ref, lse_ref = oracle.attention_rows(qd, pos, kd, vd, scale, mask, window)
    o_ref = o_ref * v_scale
    W = oracle.attention_weights_rows(qd, pos, kd, scale, mask, window)
    wmax = W.max(axis=1, keepdims=True)
    d = qd.shape[1]
    es = np.zeros(len(pos))
    for s in range(d // 64):
        cols = slice(64 * s, 64 * s + 64)
        es += np.abs(qd[:, cols]).max(axis=1) * np.abs(kd[:, cols]).max()
    # sharp inputs (integer scores, or scale 0) have exact scores
    es *= 0.0 if sharp else scale * 2.0 ** -11
    rel = (2.2 * es + 2.0 ** -10.9)[:, None] * W
    rnd = np.zeros_like(W) if sharp else np.maximum(2.0 ** -4 * W, 2.0 ** -13 * wmax)
    av = abs(v_scale)
    bound = av * ((rnd + rel) @ np.abs(vd)) + 1e-6
    var = av * av * ((rnd * rnd) @ (vd * vd)) / 3.0
    return o_ref, lse_ref, bound, var, es + 1e-5


def check(o, lse, refs, out, tag, stat=True):
    o_ref, lse_ref, bound, var, lse_tol = (np.concatenate(x) for x in zip(*refs))
    o = o.detach().to("cpu").double().numpy().reshape(o_ref.shape)
    lse = lse.detach().to("cpu").double().numpy().reshape(lse_ref.shape)
    assert np.isfinite(o).all() and np.isfinite(lse).all(), "%s: non-finite output" % tag
    lim = bound.copy()
    rvar = var.copy()
    if out != "f32":
        hu = half_ulp(np.abs(o_ref) + bound, OUT[out])
        lim += hu
        rvar += hu * hu / 3.0
    err = np.abs(o - o_ref)
    bad = err > lim
    assert not bad.any(), "%s: %d O elements over the bound, worst err %.3g vs bound %.3g" % (
        tag, int(bad.sum()), float(err[bad].max()), float(lim[bad][np.argmax(err[bad])]))
    if stat:
        mse, allowed = float(np.mean(err ** 2)), 4.0 * float(np.mean(rvar)) + 1e-12
        assert mse <= allowed, "%s: mean squared O error %.3g over %.3g" % (tag, mse, allowed)
    lerr = np.abs(lse - lse_ref)
    assert (lerr <= lse_tol).all(), "%s: lse err %.3g over %.3g" % (
        tag, float(lerr.max()), float(lse_tol[np.argmax(lerr - lse_tol)]))
    return float(err.max()), float(lerr.max())


def full_refs(q8, k8, v8, scale, v_scale, mask, window, sharp):
    """Bounds for every row of every (batch, head) slice."""
    qd, kd, vd = (oracle.decode_e4m3(x) for x in (q8, k8, v8))
    B, H, N, d = qd.shape
    H_kv = kd.shape[1]
    pos = np.arange(N)
    refs = []
    for b in range(B):
        for h in range(H):
            g = oracle.kv_head(h, H, H_kv)
            refs.append(slice_bounds(qd[b, h], pos, kd[b, g], vd[b, g], scale, mask, window,
                                     v_scale, sharp))
    return refs


# ---- building blocks ------------------------------------------------------------
def test_e4m3_product_lane_layout():
    """Lane l of both operands holds row (A) / column (B) l % 32 and
    contraction elements 32 (l / 32) .. +31; accumulator register r of lane l
    is row 8(r/4) + 4(l/32) + r%4, column l % 32.  Small integers: exact."""
    rng = np.random.default_rng(31)
    for trial, (lo, hi) in enumerate([(-4, 5), (-8, 9)]):
        say("e4m3 product probe", trial)
        A = rng.integers(lo, hi, size=(32, 64)).astype(np.float32)
        Bm = rng.integers(lo, hi, size=(64, 32)).astype(np.float32)
        la = np.empty((64, 32), np.float32)
        lb = np.empty((64, 32), np.float32)
        for l in range(64):
            la[l] = A[l % 32, 32 * (l // 32):32 * (l // 32) + 32]
            lb[l] = Bm[32 * (l // 32):32 * (l // 32) + 32, l % 32]
        a = torch.from_numpy(la).to(torch.float8_e4m3fn).view(torch.uint8).to(DEV)
        b = torch.from_numpy(lb).to(torch.float8_e4m3fn).view(torch.uint8).to(DEV)
        dres = torch.zeros(64 * 16, dtype=torch.float32, device=DEV)
        st = fa.fa_probe_mfma(3, a.data_ptr(), b.data_ptr(), dres.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
        assert st == fa.FA_OK, fa.fa_last_error()
        torch.cuda.synchronize()
        got = dres.cpu().numpy().reshape(64, 16)
        C = A.astype(np.float64) @ Bm.astype(np.float64)
        for l in range(64):
            for r in range(16):
                assert got[l, r] == C[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32], (l, r)


def test_transposing_byte_read_lane_layout():
    """ds_read_b64_tr_b8: within each 16-lane group g, lane j receives byte
    j % 8 of the 8-byte pieces addressed by lanes 16g + j/8 + 2t, t = 0..7."""
    say("tr8 probe")
    src = ((np.arange(512) * 37 + 11) % 251).astype(np.uint8)
    a = torch.from_numpy(src).to(DEV)
    dres = torch.zeros(64 * 16, dtype=torch.float32, device=DEV)
    st = fa.fa_probe_mfma(4, a.data_ptr(), a.data_ptr(), dres.data_ptr(),
                          torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK, fa.fa_last_error()
    torch.cuda.synchronize()
    got = dres.cpu().numpy()[:512].reshape(64, 8)
    for l in range(64):
        g, j = l // 16, l % 16
        want = [src[8 * (16 * g + j // 8 + 2 * t) + j % 8] for t in range(8)]
        assert list(got[l].astype(int)) == want, l


# ---- whole-tensor parity --------------------------------------------------------
MASKS = [("none", 0), ("causal", 0), ("sliding", 100)]


@pytest.mark.parametrize("mask,window", MASKS)
@pytest.mark.parametrize("H,H_kv", [(2, 2), (4, 1)])
def test_integer_scores_are_exact_up_to_the_product_sums(mask, window, H, H_kv):
    for N in (1, 77, 300, 1000):
        say("fp8 integer scores", mask, window, H, H_kv, N)
        q8, k8, v8 = si.make_qkv_e4m3_integer_scores(1, H, H_kv, N, 128, 9100 + N + H_kv)
        refs = full_refs(q8, k8, v8, LN2_F32, 1.0, mask, window, sharp=True)
        o, lse = run(q8, k8, v8, LN2_F32, 1.0, mask, window, out="f32")
        check(o, lse, refs, "f32", "int scores N=%d" % N, stat=False)


@pytest.mark.parametrize("mask,window", MASKS)
@pytest.mark.parametrize("out", ["bf16", "f16", "f32"])
def test_random_inputs_against_oracle(mask, window, out):
    for (H, H_kv), N, v_scale in zip([(2, 2), (4, 1), (4, 2), (2, 2)], [1, 65, 257, 1000],
                                     [1.0, -0.37, 2.5, 1.0]):
        say("fp8 random", mask, window, out, H, H_kv, N, v_scale)
        q8, k8, v8 = si.make_qkv_e4m3(2, H, H_kv, N, 128, 9300 + N + H)
        scale = 1.0 / math.sqrt(128)
        refs = full_refs(q8, k8, v8, scale, v_scale, mask, window, sharp=False)
        o, lse = run(q8, k8, v8, scale, v_scale, mask, window, out)
        check(o, lse, refs, out, "random N=%d H=%d/%d" % (N, H, H_kv), stat=N > 1)


def test_zero_scale_gives_exact_uniform_weights():
    """scale 0: every visible key has weight 1/|visible| and every scaled
    probability is exactly 2^3, so only the product sums remain."""
    for mask, window in MASKS:
        say("fp8 zero scale", mask)
        q8, k8, v8 = si.make_qkv_e4m3(1, 2, 2, 300, 128, 9400)
        refs = full_refs(q8, k8, v8, 0.0, 1.0, mask, window, sharp=True)
        o, lse = run(q8, k8, v8, 0.0, 1.0, mask, window, "f32")
        check(o, lse, refs, "f32", "zero scale %s" % mask, stat=False)


def test_large_scores_and_reference_resets():
    """Scaled inputs (scale 0.5 on N(0, 1) codes): peaked rows whose maximum
    moves often, exercising the exact path and the O rescale."""
    q8, k8, v8 = si.make_qkv_e4m3(1, 2, 2, 700, 128, 9500)
    for mask, window in MASKS:
        say("fp8 large scores", mask)
        refs = full_refs(q8, k8, v8, 0.5, 1.0, mask, window, sharp=False)
        o, lse = run(q8, k8, v8, 0.5, 1.0, mask, window, "f32")
        check(o, lse, refs, "f32", "large scores %s" % mask)


def test_shared_heads_equal_copied_heads_bitwise_and_calls_repeat():
    q8, k8, v8 = si.make_qkv_e4m3(2, 8, 2, 500, 128, 9600)
    kc, vc = (t.repeat_interleave(4, dim=1).contiguous() for t in (k8, v8))
    for mask, window in MASKS:
        say("fp8 copied heads", mask)
        o1, l1 = run(q8, k8, v8, 0.09, 1.0, mask, window)
        o2, l2 = run(q8, kc, vc, 0.09, 1.0, mask, window)
        o3, l3 = run(q8, k8, v8, 0.09, 1.0, mask, window)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), mask
        assert torch.equal(o1, o3) and torch.equal(l1, l3), mask


def test_torch_float8_tensors_are_accepted():
    q8, k8, v8 = si.make_qkv_e4m3(1, 2, 2, 64, 128, 9700)
    o1, l1 = run(q8, k8, v8, 0.1)
    o2, l2 = run(*(t.view(torch.float8_e4m3fn) for t in (q8, k8, v8)), 0.1)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---- the long-context shapes the benchmark times --------------------------------
def sample_rows(N, rng, extra=40):
    fixed = list(range(0, 24)) + [255, 256, 257, N // 2] + list(range(N - 24, N))
    rnd = rng.integers(0, N, size=extra).tolist()
    return np.array(sorted({r for r in fixed + rnd if 0 <= r < N}), dtype=np.int64)


@pytest.mark.parametrize("w", si.FP8_WORKLOADS, ids=[w.name for w in si.FP8_WORKLOADS])
def test_fp8_workload_sampled_rows(w):
    """Full-size launch in the benchmark's configuration; sampled rows of four
    heads against the oracle, with the bound above."""
    say("fp8 workload", w.name)
    q8, k8, v8 = si.make_workload(w)
    o, lse = run(q8, k8, v8, w.scale, 1.0, w.mask, w.window, "bf16")
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    qd_all = q8.view(torch.uint8)
    rng = np.random.default_rng(w.seed)
    for b in sorted({0, w.B - 1}):
        for h in sorted({0, 1, w.H // 2, w.H - 1}):
            rows = sample_rows(w.N, rng)
            g = oracle.kv_head(h, w.H, w.kv_heads)
            qd = oracle.decode_e4m3(qd_all[b, h][rows])
            kd, vd = oracle.decode_e4m3(k8[b, g]), oracle.decode_e4m3(v8[b, g])
            ref = slice_bounds(qd, rows, kd, vd, w.scale, w.mask, w.window, 1.0, sharp=False)
            idx = torch.from_numpy(rows).to(DEV)
            check(o[b, h].index_select(0, idx), lse[b, h].index_select(0, idx), [ref], "bf16",
                  "%s b%d h%d" % (w.name, b, h))
