"""Pins for the backward-pass oracle (oracle/attn_bwd_oracle.c): it is
checked against things other than itself.

The gradients are those of the forward definition ("FlashAttention (NL)",
section "Problemen met standaard attention"), whose intermediate P the
method recomputes rather than stores ("Memory-Optimized Flash Attention AI",
section "How it works").  Pins:
  * torch's fp64 autograd through scaled_dot_product_attention (library);
  * central finite differences of the (separately pinned) forward oracle:
    the derivative's own definition;
  * closed forms: a window of one key (o_i = v_i: dv = do, dq = dk = 0),
    constant values (o does not depend on q, k: dq = dk = 0), zero scale
    (uniform weights: dv_j = sum over the rows that see j of do_i / |V_i|);
  * invariants: the dS row sums vanish, so sum_j dk_j = 0 and a shift of
    every key leaves all gradients unchanged;
  * the row and key entry points agree with the full one;
  * planted mistakes in a private copy of the C source are caught.
"""
import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle

MASK_CASES = [("none", 0), ("causal", 0), ("sliding", 1), ("sliding", 3), ("sliding", 40)]


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


def torch_grads(q, k, v, do, scale, mask, window):
    Q, K, V = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    vis = torch.from_numpy(visible_matrix(q.shape[-2], mask, window))
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=vis, scale=scale)
    o.backward(torch.tensor(do, dtype=torch.float64))
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


@pytest.mark.parametrize("mask,window", MASK_CASES)
@pytest.mark.parametrize("d", [8, 64])
def test_matches_torch_autograd_fp64(mask, window, d):
    B, H, N = 2, 2, 53
    q, k, v, do = (rand((B, H, N, d), 31 + s) for s in range(4))
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale, mask, window)
    tq, tk, tv = torch_grads(q, k, v, do, scale, mask, window)
    np.testing.assert_allclose(dq, tq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("sliding", 2)])
def test_matches_central_differences_of_the_forward_oracle(mask, window):
    # L = sum_i <o_i, do_i>; dL/dx by (L(x + h) - L(x - h)) / 2h, every
    # element of q, k and v, with the forward oracle
    N, d, scale, h = 5, 3, 0.9, 1e-5
    q, k, v, do = (rand((N, d), 71 + s) for s in range(4))

    def loss(qq, kk, vv):
        o, _ = oracle.attention(qq, kk, vv, scale, mask, window)
        return float((o * do).sum())

    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale, mask, window)
    for x, g, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=0, atol=1e-8)


def test_window_of_one_key():
    # o_i = v_i whatever q and k are
    N, d = 40, 6
    q, k, v, do = (rand((N, d), 81 + s) for s in range(4))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.8, "sliding", 1)
    np.testing.assert_array_equal(dq, 0.0)
    np.testing.assert_array_equal(dk, 0.0)
    np.testing.assert_allclose(dv, do, rtol=0, atol=1e-15)


@pytest.mark.parametrize("mask,window", MASK_CASES)
def test_constant_values_give_no_query_or_key_gradient(mask, window):
    N, d = 37, 5
    q, k, do = rand((N, d), 91), rand((N, d), 92), rand((N, d), 93)
    v = np.broadcast_to(rand((1, d), 94), (N, d)).copy()
    dq, dk, _ = oracle.attention_bwd(q, k, v, do, 0.6, mask, window)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13


@pytest.mark.parametrize("mask,window", MASK_CASES)
def test_zero_scale_value_gradient(mask, window):
    N, d = 33, 4
    q, k, v, do = (rand((N, d), 101 + s) for s in range(4))
    _, _, dv = oracle.attention_bwd(q, k, v, do, 0.0, mask, window)
    vis = visible_matrix(N, mask, window).astype(np.float64)
    w = vis / vis.sum(axis=1, keepdims=True)  # uniform weights over each row's keys
    np.testing.assert_allclose(dv, w.T @ do, rtol=0, atol=1e-13)


@pytest.mark.parametrize("mask,window", MASK_CASES)
def test_key_gradients_sum_to_zero_and_key_shift_changes_nothing(mask, window):
    N, d = 45, 7
    q, k, v, do = (rand((N, d), 111 + s) for s in range(4))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.5, mask, window)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, rtol=0, atol=1e-12)
    u = rand((1, d), 119)
    dq2, dk2, dv2 = oracle.attention_bwd(q, k + u, v, do, 0.5, mask, window)
    np.testing.assert_allclose(dq2, dq, rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk2, dk, rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv2, dv, rtol=0, atol=1e-11)


def test_row_and_key_entries_match_the_full_entry():
    N, d = 120, 8
    q, k, v, do = (rand((N, d), 131 + s) for s in range(4))
    for mask, window in MASK_CASES:
        dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.4, mask, window)
        sel = np.array([0, 1, 2, 59, 118, 119])
        np.testing.assert_array_equal(oracle.attention_bwd_rows(q, k, v, do, sel, 0.4, mask, window),
                                      dq[sel])
        k_sel, v_sel = oracle.attention_bwd_keys(q, k, v, do, sel, 0.4, mask, window)
        np.testing.assert_array_equal(k_sel, dk[sel])
        np.testing.assert_array_equal(v_sel, dv[sel])


def test_rejects_bad_arguments():
    x = np.zeros((4, 2))
    with pytest.raises(ValueError):
        oracle.attention_bwd(x, x, x, np.zeros((5, 2)), 1.0)
    with pytest.raises(RuntimeError):
        oracle.attention_bwd_rows(x, x, x, x, [0, 9], 1.0)
    with pytest.raises(RuntimeError):
        oracle.attention_bwd_keys(x, x, x, x, [-1], 1.0)


# --------------------------------------------------------------------------
# planted mistakes
# --------------------------------------------------------------------------
SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_bwd_oracle.c")
MUTANTS = {
    "softmax_jacobian_term_dropped": ("double ds = p * (dp - D[i]);", "double ds = p * dp;"),
    "dk_scale_dropped": ("dkj[c] += scale * ds * q[i * d + c];", "dkj[c] += ds * q[i * d + c];"),
    "dv_uses_ds": ("dvj[c] += p * dout[i * d + c];", "dvj[c] += ds * dout[i * d + c];"),
    "dq_uses_v": ("for (c = 0; c < d; ++c) dqi[c] += scale * ds * k[j * d + c];",
                  "for (c = 0; c < d; ++c) dqi[c] += scale * ds * v[j * d + c];"),
    "row_D_unnormalised": ("    double p = exp(s_row[j] - m) / l;\n    double dp = 0.0;\n    for (c = 0; c < d; ++c) dp += doi[c] * v[j * d + c];\n    D += p * dp;",
                           "    double p = exp(s_row[j] - m);\n    double dp = 0.0;\n    for (c = 0; c < d; ++c) dp += doi[c] * v[j * d + c];\n    D += p * dp;"),
    "causal_transposed": ("if (mask_kind == 1) return j <= i;", "if (mask_kind == 1) return i <= j;"),
    "dp_uses_k": ("dp += dout[i * d + c] * v[j * d + c];", "dp += dout[i * d + c] * k[j * d + c];"),
}


def battery():
    cases = [
        ("torch", test_matches_torch_autograd_fp64, dict(mask="causal", window=0, d=8)),
        ("torch_sl", test_matches_torch_autograd_fp64, dict(mask="sliding", window=3, d=8)),
        ("window1", test_window_of_one_key, {}),
        ("const_v", test_constant_values_give_no_query_or_key_gradient, dict(mask="none", window=0)),
        ("zero_scale", test_zero_scale_value_gradient, dict(mask="causal", window=0)),
        ("dk_sum", test_key_gradients_sum_to_zero_and_key_shift_changes_nothing,
         dict(mask="none", window=0)),
        ("entries", test_row_and_key_entries_match_the_full_entry, {}),
    ]
    failed = []
    for name, fn, kw in cases:
        try:
            fn(**kw)
        except Exception:
            failed.append(name)
    return failed


@pytest.fixture
def swap_bwd_oracle():
    saved = oracle._bwd_lib
    yield
    oracle._bwd_lib = saved


def _compile(tmp_path, text, tag):
    src, lib = tmp_path / ("b_%s.c" % tag), tmp_path / ("b_%s.so" % tag)
    src.write_text(text)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", str(lib),
                    str(src), "-lm"], check=True)
    return str(lib)


def test_unmodified_backward_source_passes_battery(tmp_path, swap_bwd_oracle):
    oracle._bwd_lib = oracle.bind_bwd(_compile(tmp_path, open(SRC).read(), "orig"))
    assert battery() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutant_is_caught(name, tmp_path, swap_bwd_oracle):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation site not unique: %s" % name
    oracle._bwd_lib = oracle.bind_bwd(_compile(tmp_path, text.replace(old, new), name))
    assert battery(), "mutant %s passed every pin" % name


# ---- shared key/value heads ------------------------------------------------------
def torch_grads_gqa(q, k, v, do, scale, mask, window):
    Q, K, V = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    vis = torch.from_numpy(visible_matrix(q.shape[-2], mask, window))
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=vis, scale=scale,
                                                         enable_gqa=True)
    o.backward(torch.tensor(do, dtype=torch.float64))
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("sliding", 3)])
@pytest.mark.parametrize("H,H_kv", [(4, 1), (4, 2), (6, 3)])
def test_shared_heads_match_torch_autograd_fp64(mask, window, H, H_kv):
    B, N, d = 2, 29, 8
    q, do = rand((B, H, N, d), 141), rand((B, H, N, d), 142)
    k, v = rand((B, H_kv, N, d), 143), rand((B, H_kv, N, d), 144)
    dq, dk, dv = oracle.attention_bwd_gqa(q, k, v, do, 0.35, mask, window)
    tq, tk, tv = torch_grads_gqa(q, k, v, do, 0.35, mask, window)
    np.testing.assert_allclose(dq, tq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv, rtol=0, atol=1e-12)


def test_shared_heads_with_one_head_per_group_is_plain_backward():
    q, k, v, do = (rand((2, 3, 20, 5), 151 + s) for s in range(4))
    a = oracle.attention_bwd_gqa(q, k, v, do, 0.7, "causal")
    b = oracle.attention_bwd(q, k, v, do, 0.7, "causal")
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_shared_heads_equal_copied_heads_summed():
    # copying each key/value head to its g query heads and summing the
    # copies' gradients gives the shared heads' gradients
    B, H, H_kv, N, d = 1, 6, 2, 24, 4
    q, do = rand((B, H, N, d), 161), rand((B, H, N, d), 162)
    k, v = rand((B, H_kv, N, d), 163), rand((B, H_kv, N, d), 164)
    g = H // H_kv
    kc, vc = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    dq, dk, dv = oracle.attention_bwd_gqa(q, k, v, do, 0.5, "sliding", 5)
    cq, ck, cv = oracle.attention_bwd(q, kc, vc, do, 0.5, "sliding", 5)
    np.testing.assert_array_equal(dq, cq)
    np.testing.assert_allclose(dk, ck.reshape(B, H_kv, g, N, d).sum(axis=2), rtol=0, atol=1e-14)
    np.testing.assert_allclose(dv, cv.reshape(B, H_kv, g, N, d).sum(axis=2), rtol=0, atol=1e-14)
    # a round-robin grouping (h mod H_kv) is a different function: the
    # library pin above must reject it
    wrong = [oracle.attention_bwd(q[:, h], k[:, h % H_kv], v[:, h % H_kv], do[:, h], 0.5,
                                  "sliding", 5)[0] for h in range(H)]
    tq = torch_grads_gqa(q, k, v, do, 0.5, "sliding", 5)[0]
    assert not np.allclose(np.stack(wrong, axis=1), tq, atol=1e-6)


# ---------------------------------------------------------------------------
# attention_bwd_terms: the magnitude sums behind the backward's tolerance
# ---------------------------------------------------------------------------
def _terms_by_loops(q, k, v, do, scale, mask, window):
    """The five sums of attention_bwd_terms from their definitions, one
    (query, key, channel) at a time, with P from its own exponentials (no
    oracle call): the brute-force pin."""
    N, d = len(q), len(q[0])
    vis = visible_matrix(N, mask, window)
    P = [[0.0] * N for _ in range(N)]
    for i in range(N):
        s = [scale * sum(q[i][c] * k[j][c] for c in range(d)) for j in range(N)]
        m = max(s[j] for j in range(N) if vis[i, j])
        z = sum(math.exp(s[j] - m) for j in range(N) if vis[i, j])
        for j in range(N):
            P[i][j] = math.exp(s[j] - m) / z if vis[i, j] else 0.0
    o = [[sum(P[i][j] * v[j][c] for j in range(N)) for c in range(d)] for i in range(N)]
    D = [sum(do[i][c] * o[i][c] for c in range(d)) for i in range(N)]
    vmax = [max(abs(v[j][c]) for j in range(N)) for c in range(d)]
    Dm = [sum(abs(do[i][c]) * vmax[c] for c in range(d)) for i in range(N)]
    dS = [[P[i][j] * (sum(do[i][c] * v[j][c] for c in range(d)) - D[i]) for j in range(N)]
          for i in range(N)]
    aq = [[scale * sum(abs(dS[i][j]) * abs(k[j][c]) for j in range(N)) for c in range(d)]
          for i in range(N)]
    ak = [[scale * sum(abs(dS[i][j]) * abs(q[i][c]) for i in range(N)) for c in range(d)]
          for j in range(N)]
    av = [[sum(P[i][j] * abs(do[i][c]) for i in range(N)) for c in range(d)] for j in range(N)]
    rq = [[scale * math.sqrt(sum((dS[i][j] * k[j][c]) ** 2 for j in range(N))) for c in range(d)]
          for i in range(N)]
    rk = [[scale * math.sqrt(sum((dS[i][j] * q[i][c]) ** 2 for i in range(N))) for c in range(d)]
          for j in range(N)]
    rv = [[math.sqrt(sum((P[i][j] * do[i][c]) ** 2 for i in range(N))) for c in range(d)]
          for j in range(N)]
    cq = [[scale * abs(sum(P[i][j] * k[j][c] for j in range(N))) for c in range(d)]
          for i in range(N)]
    ck = [[scale * math.sqrt(sum((P[i][j] * Dm[i] * q[i][c]) ** 2 for i in range(N)))
           for c in range(d)] for j in range(N)]
    nq = [[scale * math.sqrt(sum(k[j][c] ** 2 for j in range(N) if vis[i, j])) for c in range(d)]
          for i in range(N)]
    nk = [[scale * math.sqrt(sum(q[i][c] ** 2 for i in range(N) if vis[i, j])) for c in range(d)]
          for j in range(N)]
    nv = [[math.sqrt(sum(do[i][c] ** 2 for i in range(N) if vis[i, j])) for c in range(d)]
          for j in range(N)]
    dq = [[scale * sum(dS[i][j] * k[j][c] for j in range(N)) for c in range(d)] for i in range(N)]
    dk = [[scale * sum(dS[i][j] * q[i][c] for i in range(N)) for c in range(d)] for j in range(N)]
    dv = [[sum(P[i][j] * do[i][c] for i in range(N)) for c in range(d)] for j in range(N)]
    return {n: np.array(x) for n, x in (("aq", aq), ("ak", ak), ("av", av), ("rq", rq),
                                          ("rk", rk), ("rv", rv), ("cq", cq), ("ck", ck),
                                          ("nq", nq), ("nk", nk), ("nv", nv), ("dq", dq),
                                          ("dk", dk), ("dv", dv), ("dm", Dm))}


@pytest.mark.parametrize("mask,window", MASK_CASES)
def test_bwd_terms_match_brute_force(mask, window):
    N, d = 7, 3
    q, k, v, do = (rand((N, d), 71 + s) for s in range(4))
    scale = 0.8
    o, lse = oracle.attention(q, k, v, scale, mask, window)
    got = oracle.attention_bwd_terms(q, k, v, do, o, lse, scale, mask, window)
    want = _terms_by_loops(q.tolist(), k.tolist(), v.tolist(), do.tolist(), scale, mask, window)
    assert set(got) == set(want)
    for n in want:
        np.testing.assert_allclose(got[n], want[n], rtol=1e-12, atol=1e-14, err_msg=n)
    # chosen rows and keys are the matching slices of the full result
    rows, keys = np.array([6, 0, 3]), np.array([2, 5])
    sub = oracle.attention_bwd_terms(q, k, v, do, o, lse, scale, mask, window, rows, keys)
    for n in ("aq", "rq", "cq", "nq", "dq", "dm"):
        np.testing.assert_allclose(sub[n], got[n][rows], rtol=1e-13, err_msg=n)
    for n in ("ak", "av", "rk", "rv", "ck", "nk", "nv", "dk", "dv"):
        np.testing.assert_allclose(sub[n], got[n][keys], rtol=1e-13, err_msg=n)


@pytest.mark.parametrize("mask,window", MASK_CASES)
def test_bwd_terms_bound_the_gradients(mask, window):
    """aq, ak, av are the gradients' sums with every term made non-negative:
    they bound |dq|, |dk|, |dv| (triangle inequality), and av equals dv when
    every do entry is non-negative (all weights are)."""
    N, d = 60, 8
    q, k, v, do = (rand((N, d), 91 + s) for s in range(4))
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention(q, k, v, scale, mask, window)
    t = oracle.attention_bwd_terms(q, k, v, do, o, lse, scale, mask, window)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale, mask, window)
    assert (np.abs(dq) <= t["aq"] * (1 + 1e-12) + 1e-15).all()
    assert (np.abs(dk) <= t["ak"] * (1 + 1e-12) + 1e-15).all()
    assert (np.abs(dv) <= t["av"] * (1 + 1e-12) + 1e-15).all()
    # root-sum-squares never exceed the sums of magnitudes
    assert (t["rq"] <= t["aq"] * (1 + 1e-12) + 1e-15).all()
    assert (t["rk"] <= t["ak"] * (1 + 1e-12) + 1e-15).all()
    assert (t["rv"] <= t["av"] * (1 + 1e-12) + 1e-15).all()
    # its signed sums are the gradients of the C oracle
    np.testing.assert_allclose(t["dq"], dq, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(t["dk"], dk, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(t["dv"], dv, rtol=1e-9, atol=1e-12)
    dpos = np.abs(do)
    t2 = oracle.attention_bwd_terms(q, k, v, dpos, o, lse, scale, mask, window)
    _, _, dv2 = oracle.attention_bwd(q, k, v, dpos, scale, mask, window)
    np.testing.assert_allclose(t2["av"], dv2, rtol=1e-12, atol=1e-15)
