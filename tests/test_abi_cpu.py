"""The C-ABI library on the host: it loads, exports what include/fa.h and
include/fa_diag.h declare, and rejects bad arguments before touching the
device.

Runs without a GPU.  Fake device addresses are plain integers that the
library only compares and never dereferences: every call here either fails
argument validation (pure host code) or stops at the device check.
"""
import ctypes

import pytest

import exact_io_aware_04_amd as fa

A = 1 << 20  # fake, 16-byte aligned "device" addresses, far apart
Q, K, V, O, L = A, 64 * A, 128 * A, 192 * A, 256 * A


def call(**kw):
    args = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, N=100, d=128, scale=0.1,
                mask_kind=fa.FA_MASK_CAUSAL, window=0, in_dtype=fa.FA_DTYPE_BF16,
                out_dtype=fa.FA_DTYPE_BF16, stream=None)
    args.update(kw)
    return fa.fa_fwd(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"],
                     args["H"], args["N"], args["d"], args["scale"], args["mask_kind"],
                     args["window"], args["in_dtype"], args["out_dtype"], args["stream"])


def test_library_loads_and_exports_every_declared_symbol():
    lib = fa.load()
    names = fa.declared_functions()
    assert {"fa_fwd", "fa_fwd_gqa", "fa_fwd_fp8", "fa_bwd", "fa_bwd_gqa", "fa_decode",
            "fa_decode_noalloc", "fa_decode_workspace_bytes", "fa_fwd_record_tiles",
            "fa_tile_shape", "fa_tile_map", "fa_fwd_schedule", "fa_status_string",
            "fa_last_error", "fa_probe_mfma", "fa_mfma_ceiling", "fa_bwd_kv_parts"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    # and they really are C symbols of the shared object
    so = ctypes.CDLL(fa.LIB_PATH)
    for n in names:
        assert ctypes.cast(getattr(so, n), ctypes.c_void_p).value


def test_status_strings():
    assert fa.fa_status_string(fa.FA_OK) == "FA_OK"
    assert fa.fa_status_string(fa.FA_ERR_INVALID_ARG) == "FA_ERR_INVALID_ARG"
    assert fa.fa_status_string(fa.FA_ERR_UNSUPPORTED) == "FA_ERR_UNSUPPORTED"
    assert fa.fa_status_string(fa.FA_ERR_NO_DEVICE) == "FA_ERR_NO_DEVICE"
    assert fa.fa_status_string(fa.FA_ERR_HIP) == "FA_ERR_HIP"
    assert fa.fa_status_string(99) == "FA_ERR_UNKNOWN"


INVALID = [
    dict(q=0), dict(k=0), dict(v=0), dict(o=0), dict(lse=0),
    dict(B=0), dict(H=0), dict(N=0), dict(N=-5), dict(N=1 << 30), dict(d=0),
    dict(in_dtype=7), dict(out_dtype=-1),
    dict(in_dtype=fa.FA_DTYPE_BF16, out_dtype=fa.FA_DTYPE_F16),
    dict(in_dtype=fa.FA_DTYPE_F32, out_dtype=fa.FA_DTYPE_BF16),
    dict(mask_kind=3), dict(mask_kind=fa.FA_MASK_SLIDING, window=0),
    dict(mask_kind=fa.FA_MASK_SLIDING, window=-3),
    dict(scale=float("nan")), dict(scale=float("inf")), dict(scale=-0.5),
    dict(q=Q + 8), dict(o=O + 2), dict(lse=L + 2),
    dict(o=Q + 64),             # output overlaps an input
    dict(lse=V + 1024),         # lse overlaps an input
    dict(lse=O + 4096),         # lse overlaps o
    dict(B=1 << 20, H=1 << 20, N=1 << 29, d=128),  # size overflow
]


@pytest.mark.parametrize("kw", INVALID, ids=[str(k) for k in INVALID])
def test_invalid_arguments_are_rejected_on_the_host(kw):
    st = call(**kw)
    assert st == fa.FA_ERR_INVALID_ARG, (kw, fa.fa_status_string(st))
    assert fa.fa_last_error() != ""


@pytest.mark.parametrize("d", [32, 96, 192, 512])
def test_unbuilt_head_dims_are_unsupported(d):
    assert call(d=d) == fa.FA_ERR_UNSUPPORTED
    with pytest.raises(fa.FaError):
        fa.fa_tile_shape(d, fa.FA_DTYPE_BF16)


def test_head_dim_256_is_built_for_16_bit_inputs_only():
    assert call(d=256, in_dtype=fa.FA_DTYPE_F32, out_dtype=fa.FA_DTYPE_F32) == fa.FA_ERR_UNSUPPORTED
    with pytest.raises(fa.FaError):
        fa.fa_tile_shape(256, fa.FA_DTYPE_F32)
    import torch
    if not torch.cuda.is_available():
        for dt in (fa.FA_DTYPE_BF16, fa.FA_DTYPE_F16):
            assert call(d=256, in_dtype=dt, out_dtype=dt) in (fa.FA_ERR_NO_DEVICE, fa.FA_ERR_HIP)


def test_valid_arguments_reach_the_device_check():
    # no GPU in this container: a fully valid call stops at the device check
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    st = call()
    assert st in (fa.FA_ERR_NO_DEVICE, fa.FA_ERR_HIP)
    assert fa.fa_last_error() != ""
    st = call(mask_kind=fa.FA_MASK_SLIDING, window=1, in_dtype=fa.FA_DTYPE_F32,
              out_dtype=fa.FA_DTYPE_F32, d=64)
    assert st in (fa.FA_ERR_NO_DEVICE, fa.FA_ERR_HIP)


def test_record_tiles_needs_a_buffer():
    st = fa.fa_fwd_record_tiles(Q, K, V, O, L, 1, 1, 100, 128, 0.1, 1, 0, 2, 2, None, None)
    assert st == fa.FA_ERR_INVALID_ARG


def test_probe_rejects_bad_arguments():
    assert fa.fa_probe_mfma(5, Q, K, O, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_probe_mfma(-1, Q, K, O, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_probe_mfma(0, 0, K, O, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_probe_mfma(0, Q + 4, K, O, None) == fa.FA_ERR_INVALID_ARG


def test_tile_shape():
    assert fa.fa_tile_shape(128, fa.FA_DTYPE_BF16) == (256, 32, 64)
    assert fa.fa_tile_shape(64, fa.FA_DTYPE_F16) == (256, 32, 64)
    assert fa.fa_tile_shape(64, fa.FA_DTYPE_F32) == (128, 32, 32)
    assert fa.fa_tile_shape(256, fa.FA_DTYPE_BF16) == (128, 32, 64)
    assert fa.fa_tile_shape(256, fa.FA_DTYPE_F16) == (128, 32, 64)


def test_tile_map_rejects_bad_arguments():
    buf = (ctypes.c_ubyte * 16)()
    p = ctypes.cast(buf, ctypes.c_void_p)
    lib = fa.load()
    assert lib.fa_tile_map(0, 128, 2, 0, 0, p) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_tile_map(10, 128, 2, 2, 0, p) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_tile_map(10, 128, 2, 5, 0, p) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_tile_map(10, 100, 2, 0, 0, p) == fa.FA_ERR_UNSUPPORTED
    assert lib.fa_tile_map(10, 128, 2, 0, 0, None) == fa.FA_ERR_INVALID_ARG


def test_torch_wrapper_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 1, 8, 64)
    with pytest.raises(ValueError):
        fa.attention(x, x, x)


def call_gqa(**kw):
    args = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=8, H_kv=2, N=100, d=128, scale=0.1,
                mask_kind=fa.FA_MASK_CAUSAL, window=0, in_dtype=fa.FA_DTYPE_BF16,
                out_dtype=fa.FA_DTYPE_BF16, stream=None)
    args.update(kw)
    return fa.fa_fwd_gqa(*(args[n] for n in ("q", "k", "v", "o", "lse", "B", "H", "H_kv", "N",
                                             "d", "scale", "mask_kind", "window", "in_dtype",
                                             "out_dtype", "stream")))


@pytest.mark.parametrize("kw", [dict(H_kv=0), dict(H_kv=-2), dict(H_kv=3), dict(H_kv=9),
                                dict(H=6, H_kv=4), dict(k=0), dict(N=0), dict(o=Q + 64)],
                         ids=str)
def test_shared_kv_invalid_arguments_are_rejected_on_the_host(kw):
    assert call_gqa(**kw) == fa.FA_ERR_INVALID_ARG, fa.fa_last_error()


def test_shared_kv_overlap_checks_use_the_key_value_head_count():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    # k holds B*H_kv*N*d bf16 = 2 * 100 * 128 * 2 bytes; o starting right
    # after it does not overlap, o starting inside it does
    kbytes = 2 * 100 * 128 * 2
    st = call_gqa(o=K + kbytes)
    assert st in (fa.FA_ERR_NO_DEVICE, fa.FA_ERR_HIP), fa.fa_last_error()
    assert call_gqa(o=K + kbytes - 16) == fa.FA_ERR_INVALID_ARG
    # H_kv = H and H_kv = 1 are valid
    assert call_gqa(H_kv=8) in (fa.FA_ERR_NO_DEVICE, fa.FA_ERR_HIP)
    assert call_gqa(H_kv=1) in (fa.FA_ERR_NO_DEVICE, fa.FA_ERR_HIP)


def test_torch_wrapper_rejects_mismatched_key_value_heads():
    import torch
    q = torch.zeros(1, 6, 8, 64)
    with pytest.raises(ValueError):
        fa.attention(q, torch.zeros(1, 4, 8, 64), torch.zeros(1, 4, 8, 64))
    with pytest.raises(ValueError):
        fa.attention(q, torch.zeros(1, 3, 9, 64), torch.zeros(1, 3, 9, 64))


# backward pass: q k v o dout at A-spaced fake addresses, results further on
DQ, DK, DV, DO_, LS, DL = 320 * A, 384 * A, 448 * A, 512 * A, 576 * A, 640 * A


def call_bwd(**kw):
    args = dict(q=Q, k=K, v=V, o=O, lse=LS, dout=DO_, dq=DQ, dk=DK, dv=DV, delta=DL, B=1, H=2,
                N=100, d=128, scale=0.1, mask_kind=fa.FA_MASK_CAUSAL, window=0,
                dtype=fa.FA_DTYPE_BF16, stream=None)
    args.update(kw)
    return fa.fa_bwd(*(args[n] for n in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv",
                                         "delta", "B", "H", "N", "d", "scale", "mask_kind",
                                         "window", "dtype", "stream")))


BWD_INVALID = [dict(q=0), dict(dout=0), dict(delta=0), dict(lse=0), dict(B=0), dict(N=-1),
               dict(dtype=9), dict(mask_kind=5), dict(mask_kind=fa.FA_MASK_SLIDING, window=0),
               dict(scale=float("nan")), dict(scale=-1.0), dict(dq=DQ + 8), dict(delta=DL + 2),
               dict(dq=Q + 256),          # result overlaps an input
               dict(delta=LS + 64),       # workspace overlaps lse
               dict(dk=DQ + 4096),        # two results overlap
               dict(dv=DL)]               # result overlaps the workspace


@pytest.mark.parametrize("kw", BWD_INVALID, ids=str)
def test_bwd_invalid_arguments_are_rejected_on_the_host(kw):
    assert call_bwd(**kw) == fa.FA_ERR_INVALID_ARG, fa.fa_last_error()


def test_bwd_unbuilt_cases_are_unsupported():
    assert call_bwd(dtype=fa.FA_DTYPE_F32) == fa.FA_ERR_UNSUPPORTED
    assert call_bwd(d=256) == fa.FA_ERR_UNSUPPORTED
    assert call_bwd(d=96) == fa.FA_ERR_UNSUPPORTED


def test_bwd_valid_arguments_reach_the_device_check():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    assert call_bwd() in (fa.FA_ERR_NO_DEVICE, fa.FA_ERR_HIP)
    assert call_bwd(d=64, dtype=fa.FA_DTYPE_F16, mask_kind=fa.FA_MASK_SLIDING,
                    window=7) in (fa.FA_ERR_NO_DEVICE, fa.FA_ERR_HIP)


def test_decode_workspace_bytes():
    # (H / H_kv) * Nq rows per key/value head, (d + 1) floats per row and chunk
    nb = fa.fa_decode_workspace_bytes(8, 32, 8, 1, 32768, 128)
    assert nb > 0 and nb % (8 * 32 * 1 * 129 * 4) == 0
    chunks = nb // (8 * 32 * 129 * 4)
    assert 1 <= chunks <= 32768 // 32
    assert fa.fa_decode_workspace_bytes(1, 1, 1, 1, 1, 64) == 1 * 1 * 1 * 65 * 4
    assert fa.fa_decode_workspace_bytes(1, 6, 4, 1, 100, 64) == -1   # H_kv must divide H
    assert fa.fa_decode_workspace_bytes(1, 4, 4, 9, 8, 64) == -1     # Nq > Nk


@pytest.mark.parametrize("B,H,H_kv,Nq", [(8, 32, 8, 1), (1, 8, 2, 4), (64, 8, 1, 1), (2, 32, 32, 1)])
def test_decode_workspace_bound_holds_for_every_mask(B, H, H_kv, Nq):
    """fa_decode_workspace_bytes must cover every mask and window: the chunk
    count of the split is not monotone in the number of key blocks, so a
    sliding window (fewer blocks) can need more chunks than no mask.  The
    workspace check runs on the host before any device call, so a call with
    exactly the documented size gets past it (NO_DEVICE here, never
    INVALID_ARG).  Cache sizes straddle multiples of the chunk target."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    pairs = B * H_kv
    target = min(-(-2048 // pairs), 256)
    d, dt = 128, fa.FA_DTYPE_BF16
    for m in (1, 2, 3):
        for Nk in {32 * target * m - 32, 32 * target * m - 1, 32 * target * m, 32 * target * m + 1,
                   32 * target * m + 32, 32 * target * m + 33}:
            if Nk < Nq:
                continue
            ws = fa.fa_decode_workspace_bytes(B, H, H_kv, Nq, Nk, d)
            assert ws > 0
            nq = B * H * Nq * d * 2
            nkv = B * H_kv * Nk * d * 2
            # dummy, aligned, non-overlapping device-address stand-ins
            base = 1 << 40
            qp, kp = base, base + (1 << 36)
            vp, op = kp + (1 << 36), kp + (2 << 36)
            lp, wp = kp + (3 << 36), kp + (4 << 36)
            assert nq < (1 << 36) and nkv < (1 << 36) and ws < (1 << 36)
            windows = [None, 1, 31, 32, 33, 1000, Nk - 33, Nk - 32, Nk - 1, Nk, Nk + 5]
            for w in windows:
                mask = fa.FA_MASK_CAUSAL if w is None else fa.FA_MASK_SLIDING
                if w is not None and w < 1:
                    continue
                for mk in ((mask,) if w is not None else (fa.FA_MASK_NONE, fa.FA_MASK_CAUSAL)):
                    st = fa.fa_decode(qp, kp, vp, op, lp, B, H, H_kv, Nq, Nk, d, 0.1, mk,
                                      w or 0, dt, wp, ws, None)
                    assert st == fa.FA_ERR_NO_DEVICE, (Nk, w, mk, fa.fa_last_error())


def call_decode(**kw):
    args = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=8, H_kv=2, Nq=1, Nk=1000, d=128, scale=0.1,
                mask_kind=fa.FA_MASK_CAUSAL, window=0, dtype=fa.FA_DTYPE_BF16, ws=DQ,
                ws_bytes=1 << 24, stream=None)
    args.update(kw)
    return fa.fa_decode(*(args[n] for n in ("q", "k", "v", "o", "lse", "B", "H", "H_kv", "Nq",
                                            "Nk", "d", "scale", "mask_kind", "window", "dtype",
                                            "ws", "ws_bytes", "stream")))


DEC_INVALID = [dict(q=0), dict(Nq=0), dict(Nq=1001), dict(H_kv=3), dict(H_kv=0), dict(dtype=5),
               dict(mask_kind=fa.FA_MASK_SLIDING, window=0), dict(scale=-1.0), dict(o=O + 2),
               dict(ws=0), dict(ws_bytes=16), dict(ws=DQ + 8), dict(ws=K + 64), dict(o=K + 256)]


@pytest.mark.parametrize("kw", DEC_INVALID, ids=str)
def test_decode_invalid_arguments_are_rejected_on_the_host(kw):
    assert call_decode(**kw) == fa.FA_ERR_INVALID_ARG, fa.fa_last_error()


def test_decode_unbuilt_cases_are_unsupported():
    assert call_decode(dtype=fa.FA_DTYPE_F32) == fa.FA_ERR_UNSUPPORTED
    assert call_decode(d=256) == fa.FA_ERR_UNSUPPORTED
    assert call_decode(H=8, H_kv=1, Nq=5) == fa.FA_ERR_UNSUPPORTED   # 40 rows per key/value head


def test_decode_valid_arguments_reach_the_device_check():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    assert call_decode() in (fa.FA_ERR_NO_DEVICE, fa.FA_ERR_HIP)
    assert call_decode(mask_kind=fa.FA_MASK_SLIDING, window=64, Nq=4, H=8, H_kv=1) in (
        fa.FA_ERR_NO_DEVICE, fa.FA_ERR_HIP)


# ---- 8-bit inputs (fa_fwd_fp8) ------------------------------------------------
def call_fp8(**kw):
    args = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=8, H_kv=2, N=100, d=128, scale=0.1,
                v_scale=1.0, mask_kind=fa.FA_MASK_CAUSAL, window=0,
                out_dtype=fa.FA_DTYPE_BF16, stream=None)
    args.update(kw)
    return fa.fa_fwd_fp8(*(args[n] for n in ("q", "k", "v", "o", "lse", "B", "H", "H_kv", "N",
                                             "d", "scale", "v_scale", "mask_kind", "window",
                                             "out_dtype", "stream")))


@pytest.mark.parametrize("kw", [dict(q=0), dict(lse=0), dict(B=0), dict(N=0), dict(H_kv=3),
                                dict(v_scale=float("inf")), dict(v_scale=float("nan")),
                                dict(scale=-1.0), dict(out_dtype=3), dict(out_dtype=7),
                                dict(mask_kind=fa.FA_MASK_SLIDING, window=0),
                                dict(q=Q + 8), dict(o=Q + 64)], ids=str)
def test_fp8_invalid_arguments_are_rejected_on_the_host(kw):
    assert call_fp8(**kw) == fa.FA_ERR_INVALID_ARG, fa.fa_last_error()


@pytest.mark.parametrize("d", [64, 256, 96])
def test_fp8_head_dims_other_than_128_are_unsupported(d):
    assert call_fp8(d=d) == fa.FA_ERR_UNSUPPORTED


def test_fp8_codes_are_refused_by_the_16_bit_entry_points():
    assert call(in_dtype=fa.FA_DTYPE_E4M3, out_dtype=fa.FA_DTYPE_BF16) == fa.FA_ERR_INVALID_ARG
    assert call_gqa(in_dtype=fa.FA_DTYPE_E4M3) == fa.FA_ERR_INVALID_ARG
    st = fa.fa_fwd_record_tiles(Q, K, V, O, L, 1, 1, 100, 128, 0.1, 1, 0, fa.FA_DTYPE_E4M3,
                                fa.FA_DTYPE_BF16, 4 * A, None)
    assert st == fa.FA_ERR_INVALID_ARG


def test_fp8_overlap_checks_use_one_byte_elements():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    # k holds B*H_kv*N*d E4M3 codes = 2 * 100 * 128 bytes
    kbytes = 2 * 100 * 128
    assert call_fp8(o=K + kbytes) in (fa.FA_ERR_NO_DEVICE, fa.FA_ERR_HIP), fa.fa_last_error()
    assert call_fp8(o=K + kbytes - 16) == fa.FA_ERR_INVALID_ARG


def test_fp8_valid_arguments_reach_the_device_check():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    for out in (fa.FA_DTYPE_F32, fa.FA_DTYPE_F16, fa.FA_DTYPE_BF16):
        assert call_fp8(out_dtype=out) in (fa.FA_ERR_NO_DEVICE, fa.FA_ERR_HIP)
    assert call_fp8(H_kv=8, mask_kind=fa.FA_MASK_SLIDING, window=5, v_scale=-0.5) in (
        fa.FA_ERR_NO_DEVICE, fa.FA_ERR_HIP)


def test_fp8_torch_wrapper_rejects_bad_tensors():
    import torch
    q = torch.zeros(1, 2, 8, 128, dtype=torch.uint8)
    with pytest.raises(ValueError):
        fa.attention_fp8(q, q, q)          # host tensors
    with pytest.raises(ValueError):
        fa.attention_fp8(q.float(), q, q)  # not E4M3


# ---- backward pass with shared key/value heads (fa_bwd_gqa) ---------------------
def call_bwd_gqa(**kw):
    args = dict(q=Q, k=K, v=V, o=O, lse=LS, dout=DO_, dq=DQ, dk=DK, dv=DV, delta=DL, B=1, H=8,
                H_kv=2, N=100, d=128, scale=0.1, mask_kind=fa.FA_MASK_CAUSAL, window=0,
                dtype=fa.FA_DTYPE_BF16, stream=None)
    args.update(kw)
    return fa.fa_bwd_gqa(*(args[n] for n in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv",
                                             "delta", "B", "H", "H_kv", "N", "d", "scale",
                                             "mask_kind", "window", "dtype", "stream")))


@pytest.mark.parametrize("kw", [dict(H_kv=0), dict(H_kv=3), dict(H_kv=16), dict(H_kv=-1),
                                dict(k=0), dict(dk=0), dict(N=0)], ids=str)
def test_bwd_gqa_invalid_arguments_are_rejected_on_the_host(kw):
    assert call_bwd_gqa(**kw) == fa.FA_ERR_INVALID_ARG, fa.fa_last_error()


def test_bwd_gqa_overlap_checks_use_the_key_value_head_count():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    # dk holds B*H_kv*N*d bf16 = 2 * 100 * 128 * 2 bytes: dv right after it is
    # fine, dv starting inside it overlaps
    kvbytes = 2 * 100 * 128 * 2
    assert call_bwd_gqa(dv=DK + kvbytes) in (fa.FA_ERR_NO_DEVICE, fa.FA_ERR_HIP), fa.fa_last_error()
    assert call_bwd_gqa(dv=DK + kvbytes - 16) == fa.FA_ERR_INVALID_ARG
    assert call_bwd_gqa(H_kv=8) in (fa.FA_ERR_NO_DEVICE, fa.FA_ERR_HIP)
    assert call_bwd_gqa(H_kv=1) in (fa.FA_ERR_NO_DEVICE, fa.FA_ERR_HIP)


def test_bwd_kv_parts_planner():
    """The backward's dk/dv split (host only): split when a group has at least
    8 query heads and the tiles give fewer than 4 workgroups per compute
    unit; parts = min(g / 4, ceil(4 CUs / tiles)), tiles = B H_kv ceil(N / 128)."""
    P = fa.fa_bwd_kv_parts
    # the benchmarked shapes on 256 compute units
    assert P(1, 32, 32, 16384, 256) == 1      # plain heads: g = 1
    assert P(1, 32, 8, 16384, 256) == 1       # g = 4: no room in dq for partials
    assert P(1, 32, 1, 16384, 256) == 8       # multi-query: 128 tiles, capped at g / 4
    # the GPU test shapes
    assert P(1, 32, 1, 1000, 256) == 8
    assert P(1, 9, 1, 333, 256) == 2
    assert P(1, 16, 2, 700, 256) == 2
    assert P(1, 12, 1, 129, 256) == 3
    assert P(2, 16, 1, 300, 256) == 4
    assert P(1, 8, 1, 600, 256) == 2
    # enough tiles already: no split; fewer compute units: fewer parts
    assert P(8, 32, 1, 16384, 256) == 1       # 1024 tiles = 4 per compute unit
    assert P(1, 32, 1, 16384, 64) == 2        # ceil(256 / 128)
    assert P(1, 32, 1, 16384, 1000) == 8
    for bad in ((0, 32, 1, 16, 256), (1, 32, 3, 16, 256), (1, 32, 1, 0, 256), (1, 32, 1, 16, 0),
                (1, 32, 1, 1 << 30, 256), (1, 32, 1, 2**31 - 1, 256)):
        with pytest.raises(fa.FaError):
            P(*bad)
    # the largest accepted N still plans a positive split
    assert P(1, 32, 1, (1 << 30) - 1, 256) == 1


def call_decode_noalloc(**kw):
    args = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=8, H_kv=2, Nq=1, Nk=1000, d=128, scale=0.1,
                mask_kind=fa.FA_MASK_CAUSAL, window=0, dtype=fa.FA_DTYPE_BF16, stream=None)
    args.update(kw)
    return fa.fa_decode_noalloc(*(args[n] for n in ("q", "k", "v", "o", "lse", "B", "H", "H_kv",
                                                    "Nq", "Nk", "d", "scale", "mask_kind",
                                                    "window", "dtype", "stream")))


@pytest.mark.parametrize("kw", [dict(q=0), dict(Nq=0), dict(Nq=1001), dict(H_kv=3), dict(dtype=5),
                                dict(mask_kind=fa.FA_MASK_SLIDING, window=0), dict(scale=-1.0),
                                dict(o=O + 2), dict(o=K + 256)], ids=str)
def test_decode_noalloc_checks_arguments_on_the_host(kw):
    assert call_decode_noalloc(**kw) == fa.FA_ERR_INVALID_ARG, fa.fa_last_error()


def test_decode_noalloc_rejects_sizes_beyond_its_scratch():
    """The chunk partials of fa_decode_noalloc live in an 8 MiB device array:
    larger needs are refused before any device call; sizes that fit get past
    the check (no device here)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    big = dict(B=2, H=32, H_kv=1, Nk=1 << 20, q=1 << 40, o=(1 << 40) + (1 << 32),
               k=(1 << 40) + (1 << 36), v=(1 << 40) + (2 << 36), lse=(1 << 40) + (3 << 36))
    assert fa.fa_decode_workspace_bytes(2, 32, 1, 1, 1 << 20, 128) > 8 << 20
    assert call_decode_noalloc(**big) == fa.FA_ERR_INVALID_ARG
    assert "scratch" in fa.fa_last_error()
    assert fa.fa_decode_workspace_bytes(8, 32, 8, 1, 32768, 128) <= 8 << 20
    fits = dict(B=8, H=32, H_kv=8, Nk=32768, q=1 << 40, o=(1 << 40) + (1 << 32),
                k=(1 << 40) + (1 << 36), v=(1 << 40) + (2 << 36), lse=(1 << 40) + (3 << 36))
    assert call_decode_noalloc(**fits) == fa.FA_ERR_NO_DEVICE
