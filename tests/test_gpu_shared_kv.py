"""GPU parity for query heads that share key/value heads (fa_fwd_gqa): the
multi-query attention named in "FlashAttention (NL)", section
"FlashAttention-2 (2023)" (one key/value head), and grouped heads (H / H_kv
query heads per key/value head).

* whole-tensor parity against the oracle (attention_gqa) over dtypes, head
  dims, masks, ragged N and several (H, H_kv);
* bit-identity with plain multi-head attention on key/value heads copied out
  to every query head (the same kernel arithmetic must result);
* the long-context shapes the benchmark times, sampled rows against the
  oracle one by one.
Tolerances as for fa_fwd: O max-abs <= 1e-5 (fp32 inputs) / 1e-2 (bf16,
fp16; plus half an ulp of the output dtype when O is stored in it); lse
<= 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_04_amd as fa
import oracle
import seeded_inputs as si
from tests.parity_util import compare, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()
    yield


def run(q, k, v, scale, mask="none", window=0, out_dtype=None):
    o, lse = fa.attention(q.to(DEV), k.to(DEV), v.to(DEV), scale, mask, window, out_dtype)
    torch.cuda.synchronize()
    return o, lse


HEADS = [(4, 1), (4, 2), (6, 3), (8, 4)]  # (H, H_kv)
MASKS = [("none", 0), ("causal", 0), ("sliding", 100)]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("mask,window", MASKS)
def test_shared_kv_heads_against_oracle(dtype, d, mask, window):
    if dtype == "f32" and d == 256:
        pytest.skip("head dim 256 is built for 16-bit inputs only")
    dt = DT[dtype]
    for (H, H_kv), N in zip(HEADS, [1, 65, 257, 1000]):
        say("shared kv", dtype, d, mask, window, "H", H, "H_kv", H_kv, "N", N)
        q, k, v = si.make_qkv_shared(2, H, H_kv, N, d, dtype, 8100 + N + d + H_kv)
        scale = 1.0 / math.sqrt(d)
        o_ref, lse_ref = oracle.attention_gqa(q, k, v, scale, mask, window)
        o, lse = run(q, k, v, scale, mask, window, torch.float32)
        compare(o, lse, o_ref, lse_ref, dt, "H=%d H_kv=%d N=%d fp32-out" % (H, H_kv, N))
        if dt != torch.float32:
            o, lse = run(q, k, v, scale, mask, window)
            compare(o, lse, o_ref, lse_ref, dt, "H=%d H_kv=%d N=%d dtype-out" % (H, H_kv, N))


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64), ("f32", 128), ("bf16", 256)])
@pytest.mark.parametrize("H,H_kv", [(8, 1), (8, 2), (6, 3)])
def test_shared_kv_heads_equal_copied_heads_bitwise(dtype, d, H, H_kv):
    N = 1000
    say("copied heads", dtype, d, H, H_kv)
    q, k, v = si.make_qkv_shared(2, H, H_kv, N, d, dtype, 8200 + H + H_kv)
    g = H // H_kv
    kc, vc = (t.repeat_interleave(g, dim=1).contiguous() for t in (k, v))
    for mask, window in MASKS:
        o1, l1 = run(q, k, v, 0.1, mask, window)
        o2, l2 = run(q, kc, vc, 0.1, mask, window)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), (mask, window)


def test_shared_kv_entry_point_rejects_bad_head_counts():
    q = torch.zeros(1, 6, 64, 64, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 4, 64, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        fa.attention(q, k, k)
    o = torch.empty_like(q)
    lse = torch.empty((1, 6, 64), dtype=torch.float32, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    for H_kv in (0, 4, 7, -1):
        st = fa.fa_fwd_gqa(q.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           1, 6, H_kv, 64, 64, 0.1, fa.FA_MASK_NONE, 0, fa.FA_DTYPE_BF16,
                           fa.FA_DTYPE_BF16, s)
        assert st == fa.FA_ERR_INVALID_ARG, H_kv


def sample_rows(N, rng, extra=48):
    fixed = list(range(0, 40)) + [255, 256, 257, N // 2] + list(range(N - 40, N))
    rnd = rng.integers(0, N, size=extra).tolist()
    return np.array(sorted({r for r in fixed + rnd if 0 <= r < N}), dtype=np.int64)


@pytest.mark.parametrize("w", si.SHARED_KV_WORKLOADS, ids=[w.name for w in si.SHARED_KV_WORKLOADS])
def test_shared_kv_workload_sampled_rows(w):
    """Full-size launch (the benchmark's configuration); sampled rows of four
    query heads, including two that share a key/value head, against the
    oracle one by one."""
    say("shared kv workload", w.name)
    q, k, v = si.make_workload(w)
    dt = DT[w.dtype]
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o16, lse16 = fa.attention(qd, kd, vd, w.scale, w.mask, w.window)
    o32, lse32 = fa.attention(qd, kd, vd, w.scale, w.mask, w.window, torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(o16).all() and torch.isfinite(lse16).all()
    g = w.H // w.kv_heads
    rng = np.random.default_rng(w.seed)
    for h in sorted({0, 1, w.H // 2, w.H - 1}):
        rows = sample_rows(w.N, rng)
        kv = oracle.kv_head(h, w.H, w.kv_heads)
        assert kv == h // g
        o_ref, lse_ref = oracle.attention_rows(q[0, h][rows], rows, k[0, kv], v[0, kv],
                                               w.scale, w.mask, w.window)
        idx = torch.from_numpy(rows).to(DEV)
        compare(o32[0, h].index_select(0, idx), lse32[0, h].index_select(0, idx),
                o_ref, lse_ref, dt, "%s h%d fp32-out" % (w.name, h))
        compare(o16[0, h].index_select(0, idx), lse16[0, h].index_select(0, idx),
                o_ref, lse_ref, dt, "%s h%d dtype-out" % (w.name, h))
