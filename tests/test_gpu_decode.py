"""GPU parity of decoding against a key/value cache (fa_decode) with the
oracle (oracle.attention_decode): Nq queries at the last Nq positions of Nk
cached keys, H / H_kv query heads per key/value head, split over the keys
and merged.

* shapes from one query and one key to g * Nq = 32 rows, ragged Nk, both
  16-bit types and head dims, the three masks (windows inside and beyond the
  cache);
* the decode workload the benchmark times (B=8 H=32 H_kv=8 Nq=1 Nk=32768
  d=128, causal) whole;
* determinism, workspace reuse at a smaller size, and the errors reported
  before any launch.
Tolerances as for fa_fwd: O max-abs <= 1e-2 plus half an ulp of the output
dtype, lse <= 1e-3.
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
DT = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()
    yield


def inputs(B, H, H_kv, Nq, Nk, d, dtype, seed):
    rng = np.random.default_rng(seed)
    mk = lambda shape: torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(DT[dtype])
    return mk((B, H, Nq, d)), mk((B, H_kv, Nk, d)), mk((B, H_kv, Nk, d))


SHAPES = [(1, 1, 1, 1, 1), (1, 8, 8, 1, 1), (2, 8, 2, 1, 1000), (1, 32, 8, 1, 4097),
          (2, 4, 4, 4, 777), (1, 32, 1, 1, 3000), (1, 8, 1, 4, 5000), (3, 6, 3, 3, 129),
          (1, 4, 4, 32, 32)]
MASKS = [("none", 0), ("causal", 0), ("sliding", 1), ("sliding", 100), ("sliding", 100000)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask,window", MASKS)
def test_decode_against_oracle(dtype, d, mask, window):
    for B, H, H_kv, Nq, Nk in SHAPES:
        say("decode", dtype, d, mask, window, (B, H, H_kv, Nq, Nk))
        q, k, v = inputs(B, H, H_kv, Nq, Nk, d, dtype, 7700 + Nk + Nq + d)
        scale = 1.0 / math.sqrt(d)
        o, lse = fa.attention_decode(q.to(DEV), k.to(DEV), v.to(DEV), scale, mask, window)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attention_decode(q, k, v, scale, mask, window)
        compare(o, lse, o_ref, lse_ref, DT[dtype], "decode %s" % ((B, H, H_kv, Nq, Nk),))


def test_decode_workload_whole():
    """B=8 H=32 H_kv=8 Nq=1 Nk=32768 d=128 bf16 causal: the shape and launch
    the benchmark times, every row against the oracle."""
    say("decode workload")
    q, k, v = inputs(8, 32, 8, 1, 32768, 128, "bf16", 1020)
    scale = 1.0 / math.sqrt(128)
    o, lse = fa.attention_decode(q.to(DEV), k.to(DEV), v.to(DEV), scale, "causal", 0)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_decode(q, k, v, scale, "causal", 0)
    compare(o, lse, o_ref, lse_ref, torch.bfloat16, "decode workload")


def test_decode_determinism_and_workspace_reuse():
    q, k, v = (t.to(DEV) for t in inputs(2, 8, 2, 2, 3333, 128, "bf16", 7801))
    nb = fa.fa_decode_workspace_bytes(2, 8, 2, 2, 3333, 128)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    o1, l1 = fa.attention_decode(q, k, v, 0.1, "causal", 0, workspace=ws)
    o2, l2 = fa.attention_decode(q, k, v, 0.1, "causal", 0, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # the same workspace for a smaller call, then the first call again
    qs, ks, vs = (t.to(DEV) for t in inputs(1, 4, 4, 1, 100, 128, "bf16", 7802))
    o3, l3 = fa.attention_decode(qs, ks, vs, 0.1, "causal", 0, workspace=ws)
    o4, l4 = fa.attention_decode(q, k, v, 0.1, "causal", 0, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o4, o1) and torch.equal(l4, l1)
    o_ref, lse_ref = oracle.attention_decode(qs.cpu(), ks.cpu(), vs.cpu(), 0.1, "causal", 0)
    compare(o3, l3, o_ref, lse_ref, torch.bfloat16, "smaller call")


def test_decode_errors_before_launch():
    q = torch.zeros(1, 8, 5, 128, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 1, 64, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fa.FaError) as e:   # 8 heads x 5 queries = 40 rows > 32
        fa.attention_decode(q, k, k)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    q = torch.zeros(1, 1, 65, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fa.FaError) as e:   # more queries than cached keys
        fa.attention_decode(q, k, k)
    assert e.value.status == fa.FA_ERR_INVALID_ARG
    q = torch.zeros(1, 1, 1, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fa.FaError) as e:   # workspace too small
        fa.attention_decode(q, k, k, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    assert e.value.status == fa.FA_ERR_INVALID_ARG
