"""Pins for the CPU oracle: it is checked against things other than itself.

Definition: "FlashAttention (NL)", section "Problemen met standaard
attention" (softmax(Q K^T / sqrt(d_k)) V), with the masking of section
"Samensmelting van bewerkingen in één CUDA-kernel" and the local window of
the "Sparse Attention" glossary page ("Abgrenzung & Vergleiche").

Pins used (each independent of the oracle's own code):
  * a hand-worked example (tests/golden/hand_worked_n3_d2.txt);
  * pure-Python mpmath brute force at 50 digits on tiny inputs;
  * torch's fp64 CPU scaled_dot_product_attention / logsumexp (library);
  * closed forms: constant V, zero scale (prefix / window means and ln|V_i|),
    dominant logit, window of 1, window >= N;
  * invariants: key/value permutation, query permutation, slice
    independence, power-of-two scale folding, key shift (exact lse shift),
    convex hull, and large-logit stability;
  * shared key/value heads (multi-query attention, "FlashAttention (NL)",
    section "FlashAttention-2 (2023)", and its grouped generalisation):
    torch's fp64 scaled_dot_product_attention with its own head grouping,
    mpmath brute force per query head, and a planted round-robin grouping
    that the library pin must reject.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
MASK_CASES = [("none", 0), ("causal", 0), ("sliding", 1), ("sliding", 2),
              ("sliding", 3), ("sliding", 7)]


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def visible_matrix(N, mask, window):
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    if mask == "none":
        return np.ones((N, N), dtype=bool)
    if mask == "causal":
        return j <= i
    return (j <= i) & (j > i - window)


# --------------------------------------------------------------------------
# hand-worked golden example
# --------------------------------------------------------------------------
def _expr(tok):
    if tok.startswith("ln"):
        return math.log(float(tok[2:]))
    if "/" in tok:
        a, b = tok.split("/")
        return float(a) / float(b)
    return float(tok)


def test_hand_worked_example():
    path = os.path.join(HERE, "golden", "hand_worked_n3_d2.txt")
    inputs, rows = {}, []
    for line in open(path):
        line = line.split("#")[0].split()
        if not line:
            continue
        if line[0] == "input":
            inputs[line[1]] = [_expr(t) for t in line[2:]]
        else:
            rows.append((line[0], int(line[1]), int(line[2]),
                         [_expr(t) for t in line[3:]]))
    q = np.array(inputs["q"]).reshape(3, 2)
    k = np.array(inputs["k"]).reshape(3, 2)
    v = np.array(inputs["v"]).reshape(3, 2)
    scale = inputs["scale"][0]
    assert len(rows) == 12
    for mask, window, r, (o0, o1, lse) in rows:
        o, l = oracle.attention(q, k, v, scale, mask, window)
        assert abs(o[r, 0] - o0) < 1e-13, (mask, window, r)
        assert abs(o[r, 1] - o1) < 1e-13, (mask, window, r)
        assert abs(l[r] - lse) < 1e-13, (mask, window, r)


# --------------------------------------------------------------------------
# brute force (mpmath) and library routine
# --------------------------------------------------------------------------
@pytest.mark.parametrize("N,d", [(1, 1), (2, 3), (5, 2), (7, 4), (12, 3)])
@pytest.mark.parametrize("mask,window", MASK_CASES + [("sliding", 40)])
def test_matches_mpmath_bruteforce(N, d, mask, window):
    seed = 17 * N + d + 3 * window
    q, k, v = rand((N, d), seed, 1.5), rand((N, d), seed + 1, 1.5), rand((N, d), seed + 2)
    scale = 0.7
    o, l = oracle.attention(q, k, v, scale, mask, window)
    ob, lb = oracle.bruteforce_mp(q, k, v, scale, mask, window)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, lb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mask,window", MASK_CASES + [("sliding", 64)])
@pytest.mark.parametrize("d", [16, 256])
def test_matches_torch_sdpa_fp64(mask, window, d):
    B, H, N = 2, 3, 97
    q, k, v = (torch.from_numpy(rand((B, H, N, d), s)) for s in (5, 6, 7))
    scale = 1.0 / math.sqrt(d)
    vis = torch.from_numpy(visible_matrix(N, mask, window))
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=vis, scale=scale)
    s = torch.matmul(q, k.transpose(-1, -2)) * scale
    lse_ref = torch.logsumexp(s.masked_fill(~vis, float("-inf")), dim=-1)
    o, l = oracle.attention(q, k, v, scale, mask, window)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, lse_ref.numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("mask,window", MASK_CASES)
def test_constant_values_give_that_constant(mask, window):
    # softmax rows sum to one: v_j = c for every j  =>  o_i = c
    N, d = 300, 8
    q, k = rand((2, N, d), 1, 2.0), rand((2, N, d), 2, 2.0)
    c = rand((d,), 3)
    v = np.broadcast_to(c, (2, N, d)).copy()
    o, _ = oracle.attention(q, k, v, 0.9, mask, window)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-13)


@pytest.mark.parametrize("mask,window", MASK_CASES + [("sliding", 64)])
def test_zero_scale_gives_uniform_average(mask, window):
    # scale 0 => all visible logits equal => o_i = mean of visible v_j and
    # lse_i = ln |V_i|: ln N, ln(i+1), ln min(i+1, W)
    N, d = 257, 5
    q, k, v = rand((N, d), 11), rand((N, d), 12), rand((N, d), 13)
    o, l = oracle.attention(q, k, v, 0.0, mask, window)
    csum = np.vstack([np.zeros((1, d)), np.cumsum(v, axis=0)])
    i = np.arange(N)
    if mask == "none":
        lo, hi = np.zeros(N, int), np.full(N, N)
    elif mask == "causal":
        lo, hi = np.zeros(N, int), i + 1
    else:
        lo, hi = np.maximum(0, i - window + 1), i + 1
    mean = (csum[hi] - csum[lo]) / (hi - lo)[:, None]
    np.testing.assert_allclose(o, mean, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, np.log(hi - lo), rtol=0, atol=1e-13)


@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("sliding", 3)])
def test_dominant_logit_selects_its_value(mask, window):
    # k_j = e_pi(j); q_i = alpha e_pi(t(i)) with t(i) a visible key: logit of
    # key t(i) is alpha*scale = 60, every other visible logit is 0, so
    # o_i = v_t(i) and lse_i = 60 (to within N e^-60).
    N = 40
    d = N
    rng = np.random.default_rng(21)
    pi = rng.permutation(N)
    k = np.eye(d)[pi]
    target = np.array([rng.integers(*((0, N) if mask == "none" else
                                       (max(0, i - (window if mask == "sliding" else N) + 1), i + 1)))
                       for i in range(N)])
    alpha, scale = 240.0, 0.25
    q = alpha * np.eye(d)[pi[target]]
    v = rand((N, d), 22)
    o, l = oracle.attention(q, k, v, scale, mask, window)
    np.testing.assert_allclose(o, v[target], rtol=0, atol=1e-20 + 1e-22 * N)
    np.testing.assert_allclose(l, np.full(N, 60.0), rtol=0, atol=1e-20)


def test_window_one_is_self_attention():
    N, d = 50, 6
    q, k, v = rand((N, d), 31), rand((N, d), 32), rand((N, d), 33)
    o, l = oracle.attention(q, k, v, 0.4, "sliding", 1)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_allclose(l, 0.4 * np.einsum("ic,ic->i", q, k), rtol=0, atol=1e-14)


@pytest.mark.parametrize("window", [50, 51, 1000])
def test_window_at_least_n_equals_causal(window):
    N, d = 50, 6
    q, k, v = rand((N, d), 41), rand((N, d), 42), rand((N, d), 43)
    o1, l1 = oracle.attention(q, k, v, 0.4, "sliding", window)
    o2, l2 = oracle.attention(q, k, v, 0.4, "causal", 0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def test_unmasked_permutations():
    N, d = 120, 8
    q, k, v = rand((N, d), 51), rand((N, d), 52), rand((N, d), 53)
    o, l = oracle.attention(q, k, v, 0.3)
    p = np.random.default_rng(54).permutation(N)
    o_kv, l_kv = oracle.attention(q, k[p], v[p], 0.3)
    np.testing.assert_allclose(o_kv, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l_kv, l, rtol=0, atol=1e-13)
    o_q, l_q = oracle.attention(q[p], k, v, 0.3)
    np.testing.assert_array_equal(o_q, o[p])
    np.testing.assert_array_equal(l_q, l[p])


@pytest.mark.parametrize("mask,window", MASK_CASES)
def test_slices_are_independent(mask, window):
    B, H, N, d = 2, 3, 40, 4
    q, k, v = rand((B, H, N, d), 61), rand((B, H, N, d), 62), rand((B, H, N, d), 63)
    o, l = oracle.attention(q, k, v, 0.5, mask, window)
    for b in range(B):
        for h in range(H):
            ob, lb = oracle.attention(q[b, h], k[b, h], v[b, h], 0.5, mask, window)
            np.testing.assert_array_equal(o[b, h], ob)
            np.testing.assert_array_equal(l[b, h], lb)


@pytest.mark.parametrize("c", [0.25, 2.0, 8.0])
def test_power_of_two_scale_folding(c):
    N, d = 64, 8
    q, k, v = rand((N, d), 71), rand((N, d), 72), rand((N, d), 73)
    o1, l1 = oracle.attention(q, k, v, 0.375, "causal")
    o2, l2 = oracle.attention(q * c, k, v, 0.375 / c, "causal")
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


@pytest.mark.parametrize("mask,window", MASK_CASES)
def test_key_shift_moves_lse_only(mask, window):
    # k_j -> k_j + u adds scale * q_i.u to every logit of row i: O unchanged,
    # lse_i shifted by exactly that amount
    N, d = 90, 6
    q, k, v = rand((N, d), 81), rand((N, d), 82), rand((N, d), 83)
    u = rand((d,), 84, 3.0)
    o1, l1 = oracle.attention(q, k, v, 0.6, mask, window)
    o2, l2 = oracle.attention(q, k + u, v, 0.6, mask, window)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1 + 0.6 * (q @ u), rtol=0, atol=1e-12)


@pytest.mark.parametrize("mask,window", MASK_CASES)
def test_output_in_convex_hull_of_visible_values(mask, window):
    N, d = 80, 5
    q, k, v = rand((N, d), 91, 3.0), rand((N, d), 92, 3.0), rand((N, d), 93)
    o, _ = oracle.attention(q, k, v, 1.0, mask, window)
    vis = visible_matrix(N, mask, window)
    for i in range(N):
        vv = v[vis[i]]
        assert np.all(o[i] >= vv.min(0) - 1e-14) and np.all(o[i] <= vv.max(0) + 1e-14)


def test_large_logits_stay_finite():
    # logits spanning ~2000: a softmax without the max shift would overflow;
    # shifting the keys must still move lse by exactly scale*q.u
    N, d = 64, 4
    q, k, v = rand((N, d), 101, 40.0), rand((N, d), 102, 40.0), rand((N, d), 103)
    o, l = oracle.attention(q, k, v, 1.0, "causal")
    assert np.isfinite(o).all() and np.isfinite(l).all()
    u = rand((d,), 104, 5.0)
    o2, l2 = oracle.attention(q, k + u, v, 1.0, "causal")
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-9)
    np.testing.assert_allclose(l2, l + q @ u, rtol=1e-13, atol=1e-9)


def test_rows_entry_matches_full_entry():
    N, d = 150, 8
    q, k, v = rand((N, d), 111), rand((N, d), 112), rand((N, d), 113)
    for mask, window in MASK_CASES:
        o, l = oracle.attention(q, k, v, 0.5, mask, window)
        pos = np.array([0, 1, 2, 77, 148, 149])
        orow, lrow = oracle.attention_rows(q[pos], pos, k, v, 0.5, mask, window)
        np.testing.assert_array_equal(orow, o[pos])
        np.testing.assert_array_equal(lrow, l[pos])


def test_rejects_bad_arguments():
    q = np.zeros((4, 2))
    with pytest.raises(ValueError):
        oracle.attention(q, np.zeros((5, 2)), q, 1.0)
    with pytest.raises(RuntimeError):
        oracle.attention_rows(q, [0, 1, 2, 9], q, q, 1.0)


# --------------------------------------------------------------------------
# shared key/value heads (multi-query and grouped heads)
# --------------------------------------------------------------------------
GQA_CASES = [(4, 4), (4, 2), (6, 3), (6, 2), (8, 1), (3, 1)]  # (H, H_kv)


def sdpa_gqa_fp64(q, k, v, scale, mask, window):
    """torch's fp64 CPU scaled_dot_product_attention with its own grouping of
    query heads over key/value heads (enable_gqa), and the matching lse."""
    N = q.shape[-2]
    vis = torch.from_numpy(visible_matrix(N, mask, window))
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=vis, scale=scale, enable_gqa=True)
    g = q.shape[1] // k.shape[1]
    s = torch.matmul(q, k.repeat_interleave(g, dim=1).transpose(-1, -2)) * scale
    lse = torch.logsumexp(s.masked_fill(~vis, float("-inf")), dim=-1)
    return ref.numpy(), lse.numpy()


@pytest.mark.parametrize("H,H_kv", GQA_CASES)
@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("sliding", 5)])
def test_shared_kv_heads_match_torch_sdpa_fp64(H, H_kv, mask, window):
    B, N, d = 2, 41, 8
    q = torch.from_numpy(rand((B, H, N, d), 301 + H))
    k = torch.from_numpy(rand((B, H_kv, N, d), 302 + H_kv))
    v = torch.from_numpy(rand((B, H_kv, N, d), 303 + H_kv))
    o, l = oracle.attention_gqa(q, k, v, 0.4, mask, window)
    ro, rl = sdpa_gqa_fp64(q, k, v, 0.4, mask, window)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, rl, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("sliding", 2)])
def test_multi_query_heads_match_mpmath_bruteforce(mask, window):
    # one key/value head shared by three query heads
    N, d = 6, 3
    q = rand((1, 3, N, d), 401, 1.5)
    k, v = rand((1, 1, N, d), 402, 1.5), rand((1, 1, N, d), 403)
    o, l = oracle.attention_gqa(q, k, v, 0.8, mask, window)
    for h in range(3):
        ob, lb = oracle.bruteforce_mp(q[0, h], k[0, 0], v[0, 0], 0.8, mask, window)
        np.testing.assert_allclose(o[0, h], ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l[0, h], lb, rtol=0, atol=1e-12)


def test_kv_head_grouping():
    # consecutive query heads share a key/value head
    assert [oracle.kv_head(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [oracle.kv_head(h, 6, 3) for h in range(6)] == [0, 0, 1, 1, 2, 2]
    assert {oracle.kv_head(h, 5, 1) for h in range(5)} == {0}
    assert [oracle.kv_head(h, 4, 4) for h in range(4)] == [0, 1, 2, 3]


def test_wrong_grouping_is_caught_by_the_library_pin(monkeypatch):
    # plant round-robin grouping (h mod H_kv) in the oracle: the library
    # routine's grouping must disagree
    monkeypatch.setattr(oracle, "kv_head", lambda h, H, H_kv: h % H_kv)
    B, H, H_kv, N, d = 1, 4, 2, 17, 8
    q = torch.from_numpy(rand((B, H, N, d), 501))
    k, v = torch.from_numpy(rand((B, H_kv, N, d), 502)), torch.from_numpy(rand((B, H_kv, N, d), 503))
    o, _ = oracle.attention_gqa(q, k, v, 0.4, "causal", 0)
    ro, _ = sdpa_gqa_fp64(q, k, v, 0.4, "causal", 0)
    assert np.abs(o - ro).max() > 1e-3


def test_shared_kv_heads_reject_bad_shapes():
    q = np.zeros((1, 4, 5, 2))
    with pytest.raises(ValueError):
        oracle.attention_gqa(q, np.zeros((1, 3, 5, 2)), np.zeros((1, 3, 5, 2)), 1.0)
    with pytest.raises(ValueError):
        oracle.attention_gqa(q, np.zeros((1, 2, 6, 2)), np.zeros((1, 2, 6, 2)), 1.0)
    with pytest.raises(ValueError):
        oracle.attention_gqa(q, np.zeros((1, 2, 5, 2)), np.zeros((1, 1, 5, 2)), 1.0)


# --------------------------------------------------------------------------
# decoding: a few queries at the last positions of a longer cache
# --------------------------------------------------------------------------
@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("sliding", 5), ("sliding", 40)])
@pytest.mark.parametrize("H,H_kv", [(4, 4), (4, 1), (6, 2)])
def test_decode_equals_the_last_rows_of_full_attention(mask, window, H, H_kv):
    # the decode queries are the last Nq rows of a full-length query tensor
    B, Nk, Nq, d = 2, 57, 3, 8
    qfull = rand((B, H, Nk, d), 601)
    k, v = rand((B, H_kv, Nk, d), 602), rand((B, H_kv, Nk, d), 603)
    of, lf = oracle.attention_gqa(qfull, k, v, 0.45, mask, window)
    od, ld = oracle.attention_decode(qfull[:, :, Nk - Nq:], k, v, 0.45, mask, window)
    np.testing.assert_allclose(od, of[:, :, Nk - Nq:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(ld, lf[:, :, Nk - Nq:], rtol=0, atol=1e-13)


def test_decode_with_every_query_is_plain_attention():
    q, k, v = rand((1, 2, 30, 4), 611), rand((1, 2, 30, 4), 612), rand((1, 2, 30, 4), 613)
    for mask, window in (("none", 0), ("causal", 0), ("sliding", 4)):
        od, ld = oracle.attention_decode(q, k, v, 0.7, mask, window)
        of, lf = oracle.attention(q, k, v, 0.7, mask, window)
        np.testing.assert_allclose(od, of, rtol=0, atol=1e-13)
        np.testing.assert_allclose(ld, lf, rtol=0, atol=1e-13)


def test_decode_single_query_matches_mpmath():
    # one query at the last position sees every key (causal) or the last W
    Nk, d = 9, 3
    q = rand((1, 1, 1, d), 621, 1.5)
    k, v = rand((1, 1, Nk, d), 622, 1.5), rand((1, 1, Nk, d), 623)
    for mask, window in (("causal", 0), ("sliding", 4)):
        od, ld = oracle.attention_decode(q, k, v, 0.8, mask, window)
        qfull = np.zeros((Nk, d))
        qfull[-1] = q[0, 0, 0]
        ob, lb = oracle.bruteforce_mp(qfull, k[0, 0], v[0, 0], 0.8, mask, window)
        np.testing.assert_allclose(od[0, 0, 0], ob[-1], rtol=0, atol=1e-12)
        np.testing.assert_allclose(ld[0, 0, 0], lb[-1], rtol=0, atol=1e-12)


def test_decode_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.attention_decode(np.zeros((1, 2, 5, 4)), np.zeros((1, 2, 4, 4)), np.zeros((1, 2, 4, 4)), 1.0)
    with pytest.raises(ValueError):
        oracle.attention_decode(np.zeros((1, 3, 1, 4)), np.zeros((1, 2, 4, 4)), np.zeros((1, 2, 4, 4)), 1.0)
