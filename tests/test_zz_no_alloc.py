"""fa_decode_noalloc (the decode entry point that allocates nothing: its
chunk partials live in a file-scope device array) against fa_decode with a
caller's workspace: the same plan and kernels, so the outputs must agree
bit for bit, on two calls in a row, the second on a smaller input (the
array keeps the first call's contents).  One case is also checked against
the oracle at fa_decode's tolerances."""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_04_amd as fa
import oracle
from tests.parity_util import compare, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DT = {"f16": (torch.float16, fa.FA_DTYPE_F16), "bf16": (torch.bfloat16, fa.FA_DTYPE_BF16)}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()
    yield


def _inputs(B, H, H_kv, Nq, Nk, d, dtype, seed):
    rng = np.random.default_rng(seed)
    t = DT[dtype][0]
    mk = lambda shape: torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(t).to(DEV)
    return mk((B, H, Nq, d)), mk((B, H_kv, Nk, d)), mk((B, H_kv, Nk, d))


def _run(noalloc, q, k, v, B, H, H_kv, Nq, Nk, d, mask, window, dtype):
    o = torch.full((B, H, Nq, d), float("nan"), dtype=q.dtype, device=DEV)
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=DEV)
    scale = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream().cuda_stream
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, H_kv,
            Nq, Nk, d, scale, fa.MASKS[mask], window, DT[dtype][1])
    if noalloc:
        st = fa.fa_decode_noalloc(*args, stream)
    else:
        nb = fa.fa_decode_workspace_bytes(B, H, H_kv, Nq, Nk, d)
        ws = torch.empty(nb // 4 + 64, dtype=torch.float32, device=DEV)
        st = fa.fa_decode(*args, ws.data_ptr(), nb, stream)
    assert st == fa.FA_OK, fa.fa_last_error()
    torch.cuda.synchronize()
    return o, lse


CASES = [
    # (B, H, H_kv, Nq, Nk, d, mask, window, dtype): a large call, then a smaller one
    [(8, 32, 8, 1, 32768, 128, "causal", 0, "bf16"), (2, 8, 2, 2, 3333, 128, "sliding", 1000, "bf16")],
    [(4, 16, 4, 2, 9000, 64, "none", 0, "f16"), (1, 4, 1, 1, 77, 64, "causal", 0, "f16")],
]


@pytest.mark.parametrize("pair", CASES, ids=["bf16-d128", "f16-d64"])
def test_noalloc_matches_fa_decode_twice(pair):
    for B, H, H_kv, Nq, Nk, d, mask, window, dtype in pair:
        say("noalloc", (B, H, H_kv, Nq, Nk, d, mask, window, dtype))
        assert fa.fa_decode_workspace_bytes(B, H, H_kv, Nq, Nk, d) <= 8 << 20
        q, k, v = _inputs(B, H, H_kv, Nq, Nk, d, dtype, 4242 + Nk)
        o1, l1 = _run(True, q, k, v, B, H, H_kv, Nq, Nk, d, mask, window, dtype)
        o2, l2 = _run(False, q, k, v, B, H, H_kv, Nq, Nk, d, mask, window, dtype)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
        assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all()


def test_noalloc_against_oracle():
    B, H, H_kv, Nq, Nk, d = 1, 8, 2, 3, 2000, 128
    q, k, v = _inputs(B, H, H_kv, Nq, Nk, d, "bf16", 99)
    o, lse = _run(True, q, k, v, B, H, H_kv, Nq, Nk, d, "sliding", 700, "bf16")
    o_ref, lse_ref = oracle.attention_decode(q.cpu(), k.cpu(), v.cpu(), 1.0 / math.sqrt(d),
                                             "sliding", 700)
    eo, el = compare(o, lse, o_ref, lse_ref, torch.bfloat16, "noalloc vs oracle")
    say("noalloc vs oracle: max|dO| %.3g max|dlse| %.3g" % (eo, el))


def test_noalloc_rejects_oversize_before_any_launch():
    # 2 x 32 rows x 256 chunks of (128 + 1) floats: just over 8 MiB
    B, H, H_kv, Nq, Nk, d = 2, 32, 1, 1, 1 << 20, 128
    assert fa.fa_decode_workspace_bytes(B, H, H_kv, Nq, Nk, d) > 8 << 20
    q = torch.empty((B, H, Nq, d), dtype=torch.bfloat16, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=DEV)
    st = fa.fa_decode_noalloc(q.data_ptr(), 1 << 40, (1 << 40) + (1 << 36), o.data_ptr(),
                              lse.data_ptr(), B, H, H_kv, Nq, Nk, d, 0.1, fa.FA_MASK_CAUSAL, 0,
                              fa.FA_DTYPE_BF16, None)
    assert st == fa.FA_ERR_INVALID_ARG
    assert "scratch" in fa.fa_last_error()
