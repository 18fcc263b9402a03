"""Plain CPU attention oracle (test infrastructure).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path (the HIP library
and its Python binding) never does, and this package imports nothing from it.

Two independent evaluations of the same definition live here:

* ``attention`` / ``attention_rows`` call ``attn_oracle.c`` (fp64, OpenMP,
  one score row at a time, two-pass softmax).  Its header states the
  definition and the passages of the pages it follows ("FlashAttention (NL)",
  sections "Problemen met standaard attention", "Online berekening van
  Softmax" and "Samensmelting van bewerkingen in één CUDA-kernel"; the
  "Sparse Attention" glossary page for the local window).
* ``bruteforce_mp`` evaluates the same definition in pure Python with mpmath
  at 50 significant digits, materialising the whole N x N score matrix and
  normalising exp(s) directly (no max subtraction): a different route to the
  same numbers, for tiny inputs only.

``attention_gqa`` applies ``attention`` per query head when several query
heads share one key/value head (``kv_head``: consecutive groups).

``attention_decode`` evaluates a few queries at the last positions of a
longer key/value cache (per (batch, head) through ``attention_rows``).

``decode_e4m3`` gives the value of each OCP E4M3 code (the FP8 format of
the FlashAttention-3 section of "FlashAttention (NL)" as gfx950 implements
it), written out from the format's definition; ``attention_fp8`` is
``attention_gqa`` on the decoded inputs, times the V factor: the exact
attention of the values the codes stand for.  ``attention_weights_rows``
returns the softmax weights of a few query rows (numpy, fp64), from which
the tests build the error bound of a kernel that rounds the weights.

``attention_bwd`` / ``attention_bwd_rows`` / ``attention_bwd_keys`` call
``attn_bwd_oracle.c``: the gradients dq, dk, dv of the same definition for
an output gradient do (chain rule written out, fp64); ``attention_bwd_gqa``
applies it per query head when key/value heads are shared and sums dk, dv
over each group.

Visibility of key j to query i: ``none`` all j; ``causal`` j <= i;
``sliding`` i - window < j <= i.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_BWD_SRC = os.path.join(_HERE, "attn_bwd_oracle.c")
_BWD_LIB_PATH = os.path.join(_HERE, "libbwdoracle.so")

MASKS = {"none": 0, "causal": 1, "sliding": 2}

_lib = None
_bwd_lib = None


def _gcc(src: str, out: str) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-Wall", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(force: bool = True) -> str:
    """Compile attn_oracle.c and attn_bwd_oracle.c with gcc (-O2, OpenMP, no
    fast-math) into two libraries."""
    if force or not os.path.exists(_LIB_PATH):
        _gcc(_SRC, _LIB_PATH)
    if force or not os.path.exists(_BWD_LIB_PATH):
        _gcc(_BWD_SRC, _BWD_LIB_PATH)
    return _LIB_PATH


def bind(path: str):
    """Load a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lp = ctypes.POINTER(ctypes.c_longlong)
    ll = ctypes.c_longlong
    lib.oracle_attn_f64.argtypes = [dp, dp, dp, ll, ll, ll, ctypes.c_double,
                                    ctypes.c_int, ll, dp, dp]
    lib.oracle_attn_f64.restype = ctypes.c_int
    lib.oracle_attn_rows_f64.argtypes = [dp, lp, ll, dp, dp, ll, ll,
                                         ctypes.c_double, ctypes.c_int, ll,
                                         dp, dp]
    lib.oracle_attn_rows_f64.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def bind_bwd(path: str):
    """Load a compiled backward-oracle library and declare its signatures."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lp = ctypes.POINTER(ctypes.c_longlong)
    ll, dbl, i = ctypes.c_longlong, ctypes.c_double, ctypes.c_int
    lib.oracle_attn_bwd_f64.argtypes = [dp, dp, dp, dp, ll, ll, ll, dbl, i, ll, dp, dp, dp]
    lib.oracle_attn_bwd_f64.restype = i
    lib.oracle_attn_bwd_rows_f64.argtypes = [dp, dp, dp, dp, ll, ll, dbl, i, ll, lp, ll, dp]
    lib.oracle_attn_bwd_rows_f64.restype = i
    lib.oracle_attn_bwd_keys_f64.argtypes = [dp, dp, dp, dp, ll, ll, dbl, i, ll, lp, ll, dp, dp]
    lib.oracle_attn_bwd_keys_f64.restype = i
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = bind(_LIB_PATH)
    return _lib


def _load_bwd():
    global _bwd_lib
    if _bwd_lib is None:
        if not os.path.exists(_BWD_LIB_PATH):
            build(force=False)
        _bwd_lib = bind_bwd(_BWD_LIB_PATH)
    return _bwd_lib


def _f64(x) -> np.ndarray:
    """Exact widening to a contiguous float64 numpy array (torch or numpy in)."""
    if hasattr(x, "detach"):  # torch tensor: bf16/f16/f32 -> f64 is exact
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray, ctype=ctypes.c_double):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def num_threads() -> int:
    """Threads the oracle's OpenMP regions use (OMP_NUM_THREADS honoured)."""
    return int(_load().oracle_num_threads())


def attention(q, k, v, scale: float, mask: str = "none", window: int = 0):
    """o, lse of plain attention for inputs shaped [..., N, d] (fp64 out).

    Leading dimensions (batch, heads) are independent slices.  ``lse`` is
    the natural-log normaliser ln(sum_j exp(s_ij)) over visible j.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if not (q.shape == k.shape == v.shape) or q.ndim < 2:
        raise ValueError("q, k, v must share one shape [..., N, d]")
    N, d = q.shape[-2], q.shape[-1]
    BH = int(np.prod(q.shape[:-2], dtype=np.int64)) if q.ndim > 2 else 1
    o = np.empty(q.shape, dtype=np.float64)
    lse = np.empty(q.shape[:-1], dtype=np.float64)
    rc = _load().oracle_attn_f64(_ptr(q), _ptr(k), _ptr(v), BH, N, d,
                                 float(scale), MASKS[mask], int(window),
                                 _ptr(o), _ptr(lse))
    if rc != 0:
        raise RuntimeError("oracle_attn_f64 failed (%d)" % rc)
    return o, lse


def kv_head(h: int, H: int, H_kv: int) -> int:
    """Key/value head read by query head h when H query heads share H_kv
    key/value heads (H_kv divides H): consecutive groups of H / H_kv query
    heads share one.  H_kv = 1 is multi-query attention (the extension named
    in "FlashAttention (NL)", section "FlashAttention-2 (2023)"), H_kv = H
    plain multi-head attention."""
    return h // (H // H_kv)


def attention_gqa(q, k, v, scale: float, mask: str = "none", window: int = 0):
    """o, lse (fp64) for q [B, H, N, d] and k, v [B, H_kv, N, d]: every query
    head h attends with key/value head kv_head(h, H, H_kv) of its batch
    entry, by the same definition as ``attention``."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, H, N, d] and k, v [B, H_kv, N, d]")
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if k.shape[0] != B or k.shape[2:] != (N, d) or H_kv < 1 or H % H_kv:
        raise ValueError("k, v must be [B, H_kv, N, d] with H_kv dividing H")
    o = np.empty(q.shape, dtype=np.float64)
    lse = np.empty(q.shape[:-1], dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, H_kv)
            o[b, h], lse[b, h] = attention(q[b, h], k[b, g], v[b, g], scale, mask, window)
    return o, lse


def attention_rows(q_rows, pos, k, v, scale: float, mask: str = "none",
                   window: int = 0):
    """o[R, d], lse[R] for query vectors q_rows[R, d] at positions pos[R]
    of one (batch, head) slice with keys/values k, v of shape [N, d]."""
    q_rows, k, v = _f64(q_rows), _f64(k), _f64(v)
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int64))
    R, d = q_rows.shape
    N = k.shape[0]
    if k.shape != (N, d) or v.shape != (N, d) or pos.shape != (R,):
        raise ValueError("shape mismatch")
    o = np.empty((R, d), dtype=np.float64)
    lse = np.empty((R,), dtype=np.float64)
    rc = _load().oracle_attn_rows_f64(_ptr(q_rows), _ptr(pos, ctypes.c_longlong),
                                      R, _ptr(k), _ptr(v), N, d, float(scale),
                                      MASKS[mask], int(window), _ptr(o), _ptr(lse))
    if rc != 0:
        raise RuntimeError("oracle_attn_rows_f64 failed (%d)" % rc)
    return o, lse


def attention_decode(q, k, v, scale: float, mask: str = "none", window: int = 0):
    """o, lse (fp64) for q [B, H, Nq, d] against a key/value cache k, v
    [B, H_kv, Nk, d] (Nq <= Nk): query i sits at position Nk - Nq + i, the
    last Nq positions of the sequence the cache holds, and query head h reads
    key/value head kv_head(h, H, H_kv); visibility as in ``attention`` at
    those positions.  Nq = Nk is ``attention_gqa``."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, H_kv, Nk, d]")
    B, H, Nq, d = q.shape
    H_kv, Nk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d or H_kv < 1 or H % H_kv or Nq > Nk:
        raise ValueError("k, v must be [B, H_kv, Nk, d] with H_kv dividing H and Nk >= Nq")
    pos = np.arange(Nk - Nq, Nk, dtype=np.int64)
    o = np.empty(q.shape, dtype=np.float64)
    lse = np.empty(q.shape[:-1], dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, H_kv)
            o[b, h], lse[b, h] = attention_rows(q[b, h], pos, k[b, g], v[b, g], scale, mask, window)
    return o, lse


def attention_bwd(q, k, v, do, scale: float, mask: str = "none", window: int = 0):
    """dq, dk, dv (fp64) of plain attention for inputs shaped [..., N, d],
    given the output gradient do: the chain rule of the definition, written
    out in attn_bwd_oracle.c.  Leading dimensions are independent slices."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    if not (q.shape == k.shape == v.shape == do.shape) or q.ndim < 2:
        raise ValueError("q, k, v, do must share one shape [..., N, d]")
    N, d = q.shape[-2], q.shape[-1]
    BH = int(np.prod(q.shape[:-2], dtype=np.int64)) if q.ndim > 2 else 1
    dq, dk, dv = (np.empty(q.shape, dtype=np.float64) for _ in range(3))
    rc = _load_bwd().oracle_attn_bwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(do), BH, N, d,
                                         float(scale), MASKS[mask], int(window),
                                         _ptr(dq), _ptr(dk), _ptr(dv))
    if rc != 0:
        raise RuntimeError("oracle_attn_bwd_f64 failed (%d)" % rc)
    return dq, dk, dv


def attention_bwd_gqa(q, k, v, do, scale: float, mask: str = "none", window: int = 0):
    """dq [B, H, N, d] and dk, dv [B, H_kv, N, d] (fp64) when query head h
    reads key/value head kv_head(h, H, H_kv): every query head's gradients
    by ``attention_bwd`` against its key/value head, and a key/value head's
    dk, dv the sum over the query heads that read it (the chain rule through
    the shared operand)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape or do.shape != q.shape:
        raise ValueError("q, do must be [B, H, N, d] and k, v [B, H_kv, N, d]")
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if k.shape[0] != B or k.shape[2:] != (N, d) or H_kv < 1 or H % H_kv:
        raise ValueError("k, v must be [B, H_kv, N, d] with H_kv dividing H")
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, H_kv)
            dq[b, h], dk_h, dv_h = attention_bwd(q[b, h], k[b, g], v[b, g], do[b, h], scale,
                                                 mask, window)
            dk[b, g] += dk_h
            dv[b, g] += dv_h
    return dq, dk, dv


def attention_bwd_rows(q, k, v, do, rows, scale: float, mask: str = "none",
                       window: int = 0):
    """dq[R, d] of query positions rows[R] of one [N, d] slice."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    N, d = q.shape
    if k.shape != (N, d) or v.shape != (N, d) or do.shape != (N, d) or rows.ndim != 1:
        raise ValueError("shape mismatch")
    dq = np.empty((len(rows), d), dtype=np.float64)
    rc = _load_bwd().oracle_attn_bwd_rows_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(do), N, d,
                                              float(scale), MASKS[mask], int(window),
                                              _ptr(rows, ctypes.c_longlong), len(rows),
                                              _ptr(dq))
    if rc != 0:
        raise RuntimeError("oracle_attn_bwd_rows_f64 failed (%d)" % rc)
    return dq


def attention_bwd_keys(q, k, v, do, keys, scale: float, mask: str = "none",
                       window: int = 0):
    """dk[K, d], dv[K, d] of key positions keys[K] of one [N, d] slice."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    keys = np.ascontiguousarray(np.asarray(keys, dtype=np.int64))
    N, d = q.shape
    if k.shape != (N, d) or v.shape != (N, d) or do.shape != (N, d) or keys.ndim != 1:
        raise ValueError("shape mismatch")
    dk = np.empty((len(keys), d), dtype=np.float64)
    dv = np.empty((len(keys), d), dtype=np.float64)
    rc = _load_bwd().oracle_attn_bwd_keys_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(do), N, d,
                                              float(scale), MASKS[mask], int(window),
                                              _ptr(keys, ctypes.c_longlong), len(keys),
                                              _ptr(dk), _ptr(dv))
    if rc != 0:
        raise RuntimeError("oracle_attn_bwd_keys_f64 failed (%d)" % rc)
    return dk, dv


def _codes(x) -> np.ndarray:
    """uint8 numpy array of the bytes of x (torch float8 / uint8 tensor or
    numpy / list of ints 0..255)."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu")
        if x.dtype != torch.uint8:
            x = x.view(torch.uint8)
        return x.numpy()
    a = np.asarray(x)
    if a.dtype != np.uint8:
        if np.any((a < 0) | (a > 255)):
            raise ValueError("codes must lie in 0..255")
        a = a.astype(np.uint8)
    return a


def decode_e4m3(codes) -> np.ndarray:
    """fp64 values of OCP E4M3 codes: bit 7 sign, bits 6-3 exponent field e
    (bias 7), bits 2-0 mantissa m.  e = 0: subnormal, m 2^-9 (2^(1-7) m/8);
    otherwise (1 + m/8) 2^(e-7); e = 15 with m = 7 is NaN (the format has no
    infinities, so its largest finite value is 1.75 x 2^8 = 448)."""
    c = _codes(codes).astype(np.int64)
    sign = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def attention_fp8(q8, k8, v8, scale: float, v_scale: float = 1.0, mask: str = "none",
                  window: int = 0):
    """o, lse (fp64) for E4M3 codes q8 [B, H, N, d], k8, v8 [B, H_kv, N, d]:
    every code taken at its value (``decode_e4m3``), attention as in
    ``attention_gqa``, o multiplied by v_scale.  Codes that are NaN are
    refused."""
    q, k, v = (decode_e4m3(x) for x in (q8, k8, v8))
    if np.isnan(q).any() or np.isnan(k).any() or np.isnan(v).any():
        raise ValueError("NaN codes in the inputs")
    o, lse = attention_gqa(q, k, v, scale, mask, window)
    return o * float(v_scale), lse


def attention_weights_rows(q_rows, pos, k, scale: float, mask: str = "none",
                           window: int = 0) -> np.ndarray:
    """Softmax weights W[R, N] (fp64) of query vectors q_rows[R, d] at
    positions pos[R] over the keys k[N, d] of one slice: W_rj = exp(s_rj) /
    sum_j exp(s_rj) over visible j with s = scale q k^T, 0 where j is not
    visible (a row that sees nothing is all 0).  Computed with numpy, max
    subtracted before the exponential."""
    q_rows, k = _f64(q_rows), _f64(k)
    pos = np.asarray(pos, dtype=np.int64)
    R, N = q_rows.shape[0], k.shape[0]
    s = float(scale) * (q_rows @ k.T)
    j = np.arange(N)[None, :]
    i = pos[:, None]
    if mask == "none":
        vis = np.ones((R, N), dtype=bool)
    elif mask == "causal":
        vis = j <= i
    else:
        vis = (j <= i) & (j > i - int(window))
    s = np.where(vis, s, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    mx = np.where(np.isfinite(mx), mx, 0.0)
    w = np.where(vis, np.exp(s - mx), 0.0)
    z = w.sum(axis=1, keepdims=True)
    return np.where(z > 0, w / np.where(z > 0, z, 1.0), 0.0)


def attention_bwd_terms(q, k, v, do, o, lse, scale: float, mask: str = "none",
                        window: int = 0, rows=None, keys=None) -> dict:
    """Sums over the terms of the backward pass of one [N, d] slice, the sizes
    against which its rounding is bounded (fp64, numpy).  o and lse are this
    slice's forward result from ``attention`` (fp64).  With the definitions
    of attn_bwd_oracle.c -- P_ij = exp(s_ij - lse_i) over visible pairs (0
    elsewhere), s = scale q k^T, dP_ij = <do_i, v_j>, D_i = <do_i, o_i>,
    dS_ij = P_ij (dP_ij - D_i) -- and Dm_i = sum_c |do_ic| max_j |v_jc| (an
    upper bound of sum_c |do_ic| |o_ic|: o_i is a convex combination of the
    v_j), for the query positions r in `rows` (default all) and the key
    positions t in `keys` (default all), channel c:
      dq[r, c] = scale sum_j dS_rj k_jc             the gradients themselves
      dk[t, c] = scale sum_i dS_it q_ic             (evaluated from o, lse)
      dv[t, c] = sum_i P_it do_ic
      aq, ak, av: the same sums with every term replaced by its magnitude
      rq[r, c] = scale sqrt(sum_j dS_rj^2 k_jc^2)    root-sum-squares of the
      rk[t, c] = scale sqrt(sum_i dS_it^2 q_ic^2)    terms
      rv[t, c] = sqrt(sum_i P_it^2 do_ic^2)
      cq[r, c] = scale |sum_j P_rj k_jc|             coefficient of an error
                                                     in D_r within dq[r, c]
      ck[t, c] = scale sqrt(sum_i P_it^2 Dm_i^2 q_ic^2)
      nq[r, c] = scale sqrt(sum_j vis_rj k_jc^2)     counts of the terms
      nk[t, c] = scale sqrt(sum_i vis_it q_ic^2)     (for absolute errors per
      nv[t, c] = sqrt(sum_i vis_it do_ic^2)          term)
      dm[r] = Dm_r
    |dq| <= aq, |dk| <= ak, |dv| <= av (triangle inequality)."""
    q, k, v, do, o = _f64(q), _f64(k), _f64(v), _f64(do), _f64(o)
    lse = _f64(lse)
    N, d = q.shape
    if k.shape != (N, d) or v.shape != (N, d) or do.shape != (N, d) or o.shape != (N, d) \
            or lse.shape != (N,):
        raise ValueError("q, k, v, do, o must be [N, d] and lse [N]")
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    keys = np.arange(N) if keys is None else np.asarray(keys, dtype=np.int64)
    sc = float(scale)
    D = (do * o).sum(axis=1)
    Dm = np.abs(do) @ np.abs(v).max(axis=0)

    def vis(ii, jj):
        if mask == "none":
            return np.ones((len(ii), len(jj)), dtype=bool)
        i, j = ii[:, None], jj[None, :]
        if mask == "causal":
            return j <= i
        return (j <= i) & (j > i - int(window))

    out = {}
    # query rows: full rows of P and dS
    vr = vis(rows, np.arange(N))
    P = np.where(vr, np.exp(np.where(vr, sc * (q[rows] @ k.T), 0.0) - lse[rows, None]), 0.0)
    dS = P * (do[rows] @ v.T - D[rows, None])
    out["dq"] = sc * (dS @ k)
    out["aq"] = sc * (np.abs(dS) @ np.abs(k))
    out["rq"] = sc * np.sqrt((dS * dS) @ (k * k))
    out["cq"] = sc * np.abs(P @ k)
    out["nq"] = sc * np.sqrt(vr.astype(np.float64) @ (k * k))
    out["dm"] = Dm[rows]
    # key columns: full columns of P and dS
    vc = vis(np.arange(N), keys)
    P = np.where(vc, np.exp(np.where(vc, sc * (q @ k[keys].T), 0.0) - lse[:, None]), 0.0)
    dS = P * (do @ v[keys].T - D[:, None])
    out["dk"] = sc * (dS.T @ q)
    out["dv"] = P.T @ do
    out["ak"] = sc * (np.abs(dS).T @ np.abs(q))
    out["av"] = P.T @ np.abs(do)
    out["rk"] = sc * np.sqrt((dS * dS).T @ (q * q))
    out["rv"] = np.sqrt((P * P).T @ (do * do))
    out["ck"] = sc * np.sqrt(((P * Dm[:, None]) ** 2).T @ (q * q))
    out["nk"] = sc * np.sqrt(vc.astype(np.float64).T @ (q * q))
    out["nv"] = np.sqrt(vc.astype(np.float64).T @ (do * do))
    return out


def visible(i: int, j: int, mask: str, window: int) -> bool:
    """The visibility predicate, one (query, key) pair at a time."""
    if mask == "none":
        return True
    if mask == "causal":
        return j <= i
    return i - window < j <= i


def bruteforce_mp(q, k, v, scale: float, mask: str = "none", window: int = 0,
                  dps: int = 50):
    """Pure-Python mpmath evaluation of one [N, d] slice, for tiny N and d.

    Materialises S = scale * Q K^T in full, then P_ij = exp(S_ij) / sum_j
    exp(S_ij) over visible j (masked entries have weight exactly 0), then
    O = P V and lse_i = ln sum_j exp(S_ij).  Returns float64 arrays.
    """
    import mpmath

    q, k, v = _f64(q), _f64(k), _f64(v)
    N, d = q.shape
    with mpmath.workdps(dps):
        sc = mpmath.mpf(float(scale))
        Q = [[mpmath.mpf(float(x)) for x in row] for row in q]
        K = [[mpmath.mpf(float(x)) for x in row] for row in k]
        V = [[mpmath.mpf(float(x)) for x in row] for row in v]
        S = [[sc * mpmath.fsum(Q[i][c] * K[j][c] for c in range(d))
              for j in range(N)] for i in range(N)]
        o = np.zeros((N, d))
        lse = np.full((N,), -np.inf)
        for i in range(N):
            w = [mpmath.exp(S[i][j]) if visible(i, j, mask, window) else mpmath.mpf(0)
                 for j in range(N)]
            z = mpmath.fsum(w)
            if z == 0:
                continue
            for c in range(d):
                o[i, c] = float(mpmath.fsum(w[j] * V[j][c] for j in range(N)) / z)
            lse[i] = float(mpmath.log(z))
    return o, lse
