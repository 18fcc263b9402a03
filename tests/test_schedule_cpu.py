"""The forward's work order (fa_fwd_schedule, host only): every row tile is
taken exactly once, the persistent workgroups' loads are balanced, under
the head-by-head numbering the tiles a group runs together share one head's
keys and values, and under the window-team order the members of a team
read the same key block at the same time.

The order decides speed and HBM traffic only (each tile's output depends on
its own rows), so these properties are checked here on the host; the GPU
parity tests check the outputs the same launches produce.
"""
import ctypes

import pytest

import exact_io_aware_04_amd as fa

BF16, F16, F32, E4M3 = fa.FA_DTYPE_BF16, fa.FA_DTYPE_F16, fa.FA_DTYPE_F32, fa.FA_DTYPE_E4M3
NONE, CAUSAL, SLIDING = fa.FA_MASK_NONE, fa.FA_MASK_CAUSAL, fa.FA_MASK_SLIDING

# (B, H, N, d, dtype, mask, window): the five benchmark workloads, the N
# sweep, a grouped-query case, the 8-bit and wide kernels, ragged sizes
CASES = [
    (1, 1, 128, 64, F32, NONE, 0),
    (16, 12, 1024, 64, F16, NONE, 0),
    (4, 16, 2048, 128, BF16, CAUSAL, 0),
    (1, 32, 16384, 128, BF16, CAUSAL, 0),
    (1, 32, 32768, 128, BF16, SLIDING, 4096),
    (1, 32, 2048, 128, BF16, CAUSAL, 0),
    (1, 32, 4096, 128, BF16, CAUSAL, 0),
    (1, 32, 8192, 128, BF16, CAUSAL, 0),
    (2, 8, 12288, 128, BF16, CAUSAL, 0),
    (1, 32, 16384, 128, E4M3, CAUSAL, 0),
    (1, 16, 16384, 256, BF16, CAUSAL, 0),
    (3, 5, 1000, 64, F16, CAUSAL, 0),
    (3, 5, 1000, 128, BF16, SLIDING, 300),
    (1, 1, 300, 128, BF16, CAUSAL, 0),
]
# with H_kv: every case with its own key/value heads, and shared ones
ALL = [c + (c[1],) for c in CASES] + [CASES[i] + (hkv,) for i, hkv in
                                      [(3, 8), (3, 1), (2, 4), (2, 1), (11, 1), (7, 4)]]


def case_id(c):
    return "b%dh%dkv%dn%dd%d_t%d_m%d" % (c[0], c[1], c[7], c[2], c[3], c[4], c[5])


def _rows(d, dtype):
    """Query rows per row tile (the E4M3 kernel tiles like bf16)."""
    return fa.fa_tile_shape(d, BF16 if dtype == E4M3 else dtype)[0]


def key_blocks(qt, rows, N, mask, window, bc=64):
    """Key blocks a row tile visits (mask range of its rows)."""
    r0, r1 = qt * rows, min(N, (qt + 1) * rows)
    hi = -(-N // bc) if mask == NONE else -(-r1 // bc)
    lo = 0 if mask != SLIDING else max(0, r0 - window + 1) // bc
    return hi - lo


def persistent(dtype, d):
    return dtype in (F16, BF16, E4M3) and d <= 128


@pytest.mark.parametrize("case", ALL, ids=case_id)
@pytest.mark.parametrize("cus", [256, 80])
def test_every_row_tile_exactly_once(case, cus):
    B, H, N, d, dt, mask, window, H_kv = case
    sched = fa.fa_fwd_schedule(B, H, N, d, dt, mask, cus, H_kv=H_kv, window=window)
    rows = _rows(d, dt)
    T = -(-N // rows)
    got = sorted(t for wg in sched for t in wg)
    assert got == sorted((bh, qt) for bh in range(B * H) for qt in range(T))
    if persistent(dt, d):
        assert len(sched) <= cus
        # a multiple of the 8 XCD groups when every XCD owns its own heads
        if (B * H) % 8 == 0:
            assert len(sched) % 8 == 0
    else:
        assert len(sched) == B * H * T and all(len(wg) == 1 for wg in sched)


@pytest.mark.parametrize("case", [c for c in ALL if persistent(c[4], c[3]) and c[1] * c[0] % 8 == 0],
                         ids=case_id)
def test_persistent_loads_balanced(case):
    """Per-workgroup work (key blocks visited, at least two per tile, plus
    one block's worth of tile start and output) within 3 % of the mean when
    every workgroup takes an even number of tiles (whole snake round
    pairs); the five-case list holds such cases for each numbering."""
    B, H, N, d, dt, mask, window, H_kv = case
    sched = fa.fa_fwd_schedule(B, H, N, d, dt, mask, 256, H_kv=H_kv, window=window)
    rows = _rows(d, dt)
    load = [sum(max(2, key_blocks(qt, rows, N, mask, window)) + 1 for _, qt in wg) for wg in sched]
    mean = sum(load) / len(load)
    if all(len(wg) % 2 == 0 for wg in sched):
        assert max(load) <= 1.03 * mean, (max(load), mean)


@pytest.mark.parametrize("N,H_kv,kv_per_round,heads_per_round",
                         [(16384, 32, 1, 1), (8192, 32, 1, 1), (4096, 32, 2, 2), (2048, 32, 4, 4),
                          (16384, 8, 1, 4), (16384, 1, 1, 4), (2048, 8, 1, 4)])
def test_rounds_share_key_value_heads(N, H_kv, kv_per_round, heads_per_round):
    """Causal B=1 H=32 d=128 on 256 compute units: each XCD group's 32
    workgroups take whole rounds of tiles that read one key/value head (or
    32 / (G T) of them when its G query heads have fewer than 32 tiles in
    all), so the tiles running together stream the same key/value blocks;
    the query heads of a shared key/value head alternate fastest, so a round
    holds 32 / G row tiles of each."""
    g = 32 // H_kv
    sched = fa.fa_fwd_schedule(1, 32, N, 128, BF16, CAUSAL, 256, H_kv=H_kv)
    G = len(sched)
    assert G == 256
    R = max(len(wg) for wg in sched)
    for x in range(8):
        members = [sched[gi] for gi in range(x, G, 8)]
        for k in range(R):
            tiles = [wg[k] for wg in members if k < len(wg)]
            heads = {bh for bh, _ in tiles}
            assert len({bh // g for bh in heads}) <= kv_per_round
            assert len(heads) <= heads_per_round
            assert all(h // 4 == x for h in heads)  # the group's own heads


def _timeline(wg, rows, N, window):
    """(start step, first key block, rank) of each tile of a workgroup, a tile
    taking its key blocks (at least two) plus one step (its P V-only step);
    the tile start and output cost the same for every tile."""
    t, out = 0, []
    for _, qt in wg:
        lo = max(0, qt * rows - window + 1) // 64
        out.append((t, lo, qt))
        t += max(2, key_blocks(qt, rows, N, SLIDING, window)) + 1
    return out


@pytest.mark.parametrize("B,H,H_kv,N,window,cus,S",
                         [(1, 32, 32, 32768, 4096, 256, 16), (1, 32, 8, 32768, 4096, 256, 16),
                          (2, 32, 32, 16384, 2048, 256, 8), (1, 64, 64, 8192, 1024, 128, 4),
                          (1, 12, 12, 8192, 1024, 24, 4), (1, 32, 32, 4096, 4096, 256, 16)])
def test_sliding_window_teams_stream_one_block(B, H, H_kv, N, window, cus, S):
    """Windows of S row tiles: the group's workgroups form teams of S; once
    each member has finished the first tile of a head (or before the last
    one of an odd head), every member of a team reads the same key block at
    the same step, and each member's load is the same."""
    sched = fa.fa_fwd_schedule(B, H, N, 128, BF16, SLIDING, cus, H_kv=H_kv, window=window)
    rows = 256
    T = N // rows
    G = len(sched)
    n_groups = 8 if (B * H) % 8 == 0 else 1
    J = G // n_groups
    M = T // S
    loads = set()
    for x in range(n_groups):
        members = [sched[gi] for gi in range(x, G, n_groups)]
        for team in range(J // S):
            lines = [_timeline(members[team * S + i], rows, N, window) for i in range(S)]
            assert len({len(tl) for tl in lines}) == 1
            for k in range(len(lines[0])):
                hh, kk = divmod(k, M)
                ramp = kk == 0 if hh % 2 == 0 else kk == M - 1
                heads = {members[team * S + i][k][0] for i in range(S)}
                assert len(heads) == 1  # one head per team at a time
                if not ramp:
                    # start step - first key block equal across the team
                    assert len({t - lo for t, lo, _ in (tl[k] for tl in lines)}) == 1
                else:
                    assert all(tl[k][2] < S for tl in lines)
            for i in range(S):
                wg = members[team * S + i]
                loads.add(sum(max(2, key_blocks(qt, rows, N, SLIDING, window)) + 1 for _, qt in wg))
    assert len(loads) == 1


@pytest.mark.parametrize("H,N,window", [(32, 32768, 4000), (32, 32768, 2048), (24, 32768, 4096),
                                        (32, 32000, 4096)])
def test_sliding_window_without_teams_keeps_heads_fastest(H, N, window):
    """Windows that are not a whole number of row tiles, teams that would get
    an odd number of heads, or N not a multiple of the row tile: heads
    numbered fastest, the short tiles at each head's start in the last
    rounds, spread over every workgroup."""
    sched = fa.fa_fwd_schedule(1, H, N, 128, BF16, SLIDING, 256, window=window)
    first = [wg[0] for wg in sched]
    T = -(-N // 256)
    assert len({bh for bh, _ in first}) == min(H, len(sched))
    assert all(qt >= T - 16 for _, qt in first)


def test_schedule_rejects_bad_arguments():
    lib = fa.load()
    G, R = ctypes.c_int(0), ctypes.c_int(0)
    g, r = ctypes.byref(G), ctypes.byref(R)
    assert lib.fa_fwd_schedule(0, 1, 1, 10, 128, BF16, 0, 0, 256, g, r, None, 0) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_fwd_schedule(1, 1, 1, 10, 128, BF16, 7, 0, 256, g, r, None, 0) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_fwd_schedule(1, 1, 1, 10, 128, BF16, 0, 0, 0, g, r, None, 0) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_fwd_schedule(1, 1, 1, 10, 100, BF16, 0, 0, 256, g, r, None, 0) == fa.FA_ERR_UNSUPPORTED
    assert lib.fa_fwd_schedule(1, 1, 1, 10, 128, 9, 0, 0, 256, g, r, None, 0) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_fwd_schedule(1, 1, 1, 10, 128, BF16, 0, 0, 256, None, r, None, 0) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_fwd_schedule(1, 1, 1, 1 << 30, 128, BF16, 0, 0, 256, g, r, None, 0) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_fwd_schedule(1, 4, 3, 10, 128, BF16, 0, 0, 256, g, r, None, 0) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_fwd_schedule(1, 4, 0, 10, 128, BF16, 0, 0, 256, g, r, None, 0) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_fwd_schedule(1, 2, 2, 1000, 128, BF16, 1, 0, 256, g, r, None, 0) == fa.FA_OK
    assert lib.fa_fwd_schedule(1, 2, 2, 1000, 128, BF16, 2, 0, 256, g, r, None, 0) == fa.FA_ERR_INVALID_ARG
    buf = (ctypes.c_int * 4)()
    assert lib.fa_fwd_schedule(1, 2, 2, 1000, 128, BF16, 1, 0, 256, g, r,
                               ctypes.cast(buf, ctypes.c_void_p), 4) == fa.FA_ERR_INVALID_ARG
