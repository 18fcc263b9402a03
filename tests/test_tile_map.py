"""The host tile map (fa_tile_map, the same classifier the kernels run)
against a brute-force map built element by element from the oracle's
visibility predicate.

A block of rows x keys is SKIP if no (query, key) pair in it is visible,
FULL if every pair is visible and every key exists (< N), else PARTIAL.
"""
import numpy as np
import pytest

import exact_io_aware_04_amd as fa
import oracle


def brute_map(N, rows, keys, mask, window):
    R, C = -(-N // rows), -(-N // keys)
    Np = max(R * rows, C * keys)
    i = np.arange(Np)[:, None]
    j = np.arange(Np)[None, :]
    if mask == "none":
        vis = np.ones((Np, Np), bool)
    elif mask == "causal":
        vis = j <= i
    else:
        vis = (j <= i) & (j > i - window)
    vis = vis & (j < N)
    out = np.zeros((R, C), np.uint8)
    for rb in range(R):
        r0, r1 = rb * rows, min(N, rb * rows + rows)
        for kb in range(C):
            blk = vis[r0:r1, kb * keys:(kb + 1) * keys]
            if not blk.any():
                out[rb, kb] = fa.FA_TILE_SKIP
            elif blk.all():
                out[rb, kb] = fa.FA_TILE_FULL
            else:
                out[rb, kb] = fa.FA_TILE_PARTIAL
    return out


def test_brute_map_uses_the_oracle_predicate():
    # the vectorised predicate above is the oracle's, pair by pair
    for mask, w in [("none", 0), ("causal", 0), ("sliding", 3)]:
        for i in range(9):
            for j in range(9):
                want = oracle.visible(i, j, mask, w)
                got = (mask == "none") or (j <= i and (mask == "causal" or j > i - w))
                assert want == got


NS = [1, 2, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 257, 1000]
CASES = [("none", 0), ("causal", 0)] + [("sliding", w) for w in
                                        (1, 2, 31, 32, 33, 63, 64, 65, 100, 4096)]


@pytest.mark.parametrize("dtype", [fa.FA_DTYPE_BF16, fa.FA_DTYPE_F32])
@pytest.mark.parametrize("mask,window", CASES)
def test_tile_map_matches_brute_force(dtype, mask, window):
    _, rows, keys = fa.fa_tile_shape(128, dtype)
    for N in NS:
        got = np.array(fa.fa_tile_map(N, 128, dtype, fa.MASKS[mask], window), np.uint8)
        want = brute_map(N, rows, keys, mask, window)
        np.testing.assert_array_equal(got, want, err_msg="N=%d" % N)


def test_long_context_tile_counts():
    # causal N=16384: 512 row blocks of 32 x 256 key blocks of 64; the
    # processed (non-SKIP) blocks are the lower triangle at block level.
    m = np.array(fa.fa_tile_map(16384, 128, fa.FA_DTYPE_BF16, fa.FA_MASK_CAUSAL, 0))
    assert m.shape == (512, 256)
    rb = np.arange(512)[:, None]
    kb = np.arange(256)[None, :]
    np.testing.assert_array_equal(m != fa.FA_TILE_SKIP, kb * 64 <= rb * 32 + 31)
    assert (m == fa.FA_TILE_PARTIAL).sum() == 512  # one diagonal block per row block
    # sliding window W=4096 over N=32768: at most 66 key blocks per row block
    s = np.array(fa.fa_tile_map(32768, 128, fa.FA_DTYPE_BF16, fa.FA_MASK_SLIDING, 4096))
    assert (s != fa.FA_TILE_SKIP).sum(axis=1).max() <= 66
    for rb in (0, 127, 128, 200, 1023):
        r0, r1 = 32 * rb, 32 * rb + 32
        first, last = max(0, r0 - 4096 + 1) // 64, (r1 - 1) // 64
        assert (s[rb] != fa.FA_TILE_SKIP).sum() == last - first + 1
