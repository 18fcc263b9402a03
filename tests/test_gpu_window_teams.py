"""Sliding windows of whole row tiles run in window teams (fa_persist_tile_of):
the launch's work order differs from every other shape's, so its outputs
are checked here against the oracle at shapes where that order is in use
on this device -- the 16-bit kernel with shared key/value heads over the
whole output, and the E4M3 kernel on sampled rows of every head.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_04_amd as fa
import oracle
import seeded_inputs as si
from tests.parity_util import compare, say
from tests.test_gpu_fp8 import check, sample_rows, slice_bounds

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ROWS = 256  # query rows per persistent workgroup (d = 128)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()
    yield


def require_teams(B, H, H_kv, N, dtype_code, window):
    """Skip unless this device's launch numbers the tiles in window teams:
    every workgroup's first tile is one of the S short ones and its ranks
    then advance by S (S = window / row tile)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sched = fa.fa_fwd_schedule(B, H, N, 128, dtype_code, fa.FA_MASK_SLIDING, cus, H_kv=H_kv,
                               window=window)
    S = window // ROWS
    ok = all(wg and wg[0][1] < S and all(b[1] - a[1] == S for a, b in zip(wg, wg[1:])
                                          if a[0] == b[0] and b[1] >= S)
             for wg in sched)
    if not ok:
        pytest.skip("window teams not used with %d compute units" % cus)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_window_teams_shared_heads_whole_tensor(dtype):
    """B=1 H=32 H_kv=8 N=8192, window 4096 (16 row tiles): every element of O
    (fp32 and input-type output) and lse against the fp64 oracle."""
    B, H, H_kv, N, W = 1, 32, 8, 8192, 4096
    code = fa.FA_DTYPE_BF16 if dtype == "bf16" else fa.FA_DTYPE_F16
    require_teams(B, H, H_kv, N, code, W)
    say("window teams", dtype, B, H, H_kv, N, W)
    q, k, v = si.make_qkv_shared(B, H, H_kv, N, 128, dtype, 8700 + (dtype == "f16"))
    scale = 1.0 / math.sqrt(128)
    o_ref, lse_ref = oracle.attention_gqa(q, k, v, scale, "sliding", W)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float16
    for out in (torch.float32, None):
        o, lse = fa.attention(q.to(DEV), k.to(DEV), v.to(DEV), scale, "sliding", W, out)
        torch.cuda.synchronize()
        e, le = compare(o, lse, o_ref, lse_ref, dt, "window teams %s out=%s" % (dtype, out))
        print("window teams %s out=%s: max|dO| %.3g max|dlse| %.3g" % (dtype, out, e, le))


def test_window_teams_e4m3_sampled_rows():
    """E4M3, B=1 H=32 N=16384, window 4096: sampled rows (tile edges
    included) of every head against the oracle, within the rounding bound
    of the E4M3 parity tests."""
    B, H, H_kv, N, W = 1, 32, 32, 16384, 4096
    require_teams(B, H, H_kv, N, fa.FA_DTYPE_E4M3, W)
    say("window teams e4m3", B, H, N, W)
    q8, k8, v8 = si.make_qkv_e4m3(B, H, H_kv, N, 128, 8710)
    scale = 1.0 / math.sqrt(128)
    o, lse = fa.attention_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), scale, 1.0, "sliding", W,
                              torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(8710)
    qd_all = q8.view(torch.uint8)
    for h in range(H):
        rows = sample_rows(N, rng, extra=16)
        g = oracle.kv_head(h, H, H_kv)
        qd = oracle.decode_e4m3(qd_all[0, h][rows])
        kd, vd = oracle.decode_e4m3(k8[0, g]), oracle.decode_e4m3(v8[0, g])
        ref = slice_bounds(qd, rows, kd, vd, scale, "sliding", W, 1.0, sharp=False)
        idx = torch.from_numpy(rows).to(DEV)
        check(o[0, h].index_select(0, idx), lse[0, h].index_select(0, idx), [ref], "bf16",
              "window teams e4m3 h%d" % h)
