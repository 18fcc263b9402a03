"""Python binding of libfa.so: the fused exact attention forward pass on
gfx950 (MI355X).

The functions named like the C ABI (``fa_fwd``, ``fa_fwd_gqa``, ``fa_fwd_fp8``, ``fa_bwd_gqa``, ``fa_decode``,
``fa_decode_workspace_bytes``, ``fa_decode_noalloc``, ``fa_bwd``, ``fa_fwd_record_tiles``,
``fa_tile_shape``, ``fa_tile_map``, ``fa_fwd_schedule``, ``fa_status_string``, ``fa_last_error``,
``fa_probe_mfma``, ``fa_mfma_ceiling``) only marshal arguments: pointers are plain integers
(device addresses, e.g. ``tensor.data_ptr()``), the stream is a hipStream_t
handle (``torch.cuda.current_stream().cuda_stream``), and every step of the
computation runs in the library's kernels.  ``attention`` is the torch-facing
convenience: it allocates o and lse with torch on the inputs' device and
calls ``fa_fwd`` on the current stream; ``attention_fp8``, ``attention_bwd``
and ``attention_decode`` do the same for the other entry points.

There is no fallback: if libfa.so is not built, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import math
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "fa.h")
# every header of the library: the method calls (fa.h) and the diagnostics
# and host-side planners (fa_diag.h)
HEADER_PATHS = (HEADER_PATH, os.path.join(os.path.dirname(_PKG), "include", "fa_diag.h"))

FA_DTYPE_F32, FA_DTYPE_F16, FA_DTYPE_BF16, FA_DTYPE_E4M3 = 0, 1, 2, 3
FA_MASK_NONE, FA_MASK_CAUSAL, FA_MASK_SLIDING = 0, 1, 2
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_NO_DEVICE, FA_ERR_HIP = range(5)
FA_TILE_SKIP, FA_TILE_FULL, FA_TILE_PARTIAL = 0, 1, 2

MASKS = {"none": FA_MASK_NONE, "causal": FA_MASK_CAUSAL, "sliding": FA_MASK_SLIDING}


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (where, fa_status_string(status), fa_last_error()))


_lib = None


def load():
    """Load libfa.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libfa.so is not built at %s; run __graft_entry__.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    ip = ctypes.POINTER(ctypes.c_int)
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, i, vp]
    lib.fa_fwd_gqa.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, f, i, i, i, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_bwd.argtypes = [vp] * 10 + [i, i, i, i, f, i, i, i, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_gqa.argtypes = [vp] * 10 + [i, i, i, i, i, f, i, i, i, vp]
    lib.fa_bwd_gqa.restype = i
    lib.fa_decode_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.fa_decode_workspace_bytes.restype = ctypes.c_longlong
    lib.fa_decode.argtypes = [vp] * 5 + [i] * 6 + [f, i, i, i, vp, ctypes.c_longlong, vp]
    lib.fa_decode.restype = i
    lib.fa_decode_noalloc.argtypes = [vp] * 5 + [i] * 6 + [f, i, i, i, vp]
    lib.fa_decode_noalloc.restype = i
    lib.fa_fwd_record_tiles.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i, i, vp, vp]
    lib.fa_fwd_record_tiles.restype = i
    lib.fa_tile_shape.argtypes = [i, i, ip, ip, ip]
    lib.fa_bwd_kv_parts.restype = i
    lib.fa_bwd_kv_parts.argtypes = [i, i, i, i, i, ip]
    lib.fa_tile_shape.restype = i
    lib.fa_tile_map.argtypes = [i, i, i, i, i, vp]
    lib.fa_tile_map.restype = i
    lib.fa_fwd_schedule.argtypes = [i, i, i, i, i, i, i, i, i, ip, ip, vp, ctypes.c_longlong]
    lib.fa_fwd_schedule.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    lib.fa_probe_mfma.argtypes = [i, vp, vp, vp, vp]
    lib.fa_probe_mfma.restype = i
    lib.fa_mfma_ceiling.argtypes = [i, i, vp, vp, vp]
    lib.fa_mfma_ceiling.restype = i
    _lib = lib
    return lib


def declared_functions():
    """Names of the functions include/fa.h and include/fa_diag.h declare."""
    text = "".join(open(h).read() for h in HEADER_PATHS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


# ---- raw C-ABI mirrors ------------------------------------------------------
def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, mask_kind, window, in_dtype,
           out_dtype, stream) -> int:
    return load().fa_fwd(q, k, v, o, lse, B, H, N, d, scale, mask_kind, window,
                         in_dtype, out_dtype, stream)


def fa_fwd_gqa(q, k, v, o, lse, B, H, H_kv, N, d, scale, mask_kind, window, in_dtype,
               out_dtype, stream) -> int:
    return load().fa_fwd_gqa(q, k, v, o, lse, B, H, H_kv, N, d, scale, mask_kind, window,
                             in_dtype, out_dtype, stream)


def fa_fwd_fp8(q, k, v, o, lse, B, H, H_kv, N, d, scale, v_scale, mask_kind, window,
               out_dtype, stream) -> int:
    return load().fa_fwd_fp8(q, k, v, o, lse, B, H, H_kv, N, d, scale, v_scale, mask_kind,
                             window, out_dtype, stream)


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, mask_kind, window,
           dtype, stream) -> int:
    return load().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, mask_kind,
                         window, dtype, stream)


def fa_bwd_gqa(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, H_kv, N, d, scale, mask_kind,
               window, dtype, stream) -> int:
    return load().fa_bwd_gqa(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, H_kv, N, d, scale,
                             mask_kind, window, dtype, stream)


def fa_decode_workspace_bytes(B, H, H_kv, Nq, Nk, d) -> int:
    return load().fa_decode_workspace_bytes(B, H, H_kv, Nq, Nk, d)


def fa_decode(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, mask_kind, window, dtype,
              workspace, workspace_bytes, stream) -> int:
    return load().fa_decode(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, mask_kind, window,
                            dtype, workspace, workspace_bytes, stream)


def fa_decode_noalloc(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, mask_kind, window, dtype,
                      stream) -> int:
    return load().fa_decode_noalloc(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, mask_kind,
                                    window, dtype, stream)


def fa_fwd_record_tiles(q, k, v, o, lse, B, H, N, d, scale, mask_kind, window,
                        in_dtype, out_dtype, tiles, stream) -> int:
    return load().fa_fwd_record_tiles(q, k, v, o, lse, B, H, N, d, scale, mask_kind,
                                      window, in_dtype, out_dtype, tiles, stream)


def fa_bwd_kv_parts(B: int, H: int, H_kv: int, N: int, compute_units: int) -> int:
    """Workgroups per key tile of the backward's dk/dv pass; raises on error."""
    parts = ctypes.c_int()
    st = load().fa_bwd_kv_parts(B, H, H_kv, N, compute_units, ctypes.byref(parts))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_kv_parts")
    return parts.value


def fa_tile_shape(d: int, in_dtype: int):
    """(rows_per_workgroup, rows_per_wave, keys_per_block); raises on error."""
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    st = load().fa_tile_shape(d, in_dtype, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
    if st != FA_OK:
        raise FaError(st, "fa_tile_shape")
    return a.value, b.value, c.value


def fa_tile_map(N: int, d: int, in_dtype: int, mask_kind: int, window: int):
    """Host tile map as a list of rows (one per row block) of FA_TILE_*."""
    _, rw, bc = fa_tile_shape(d, in_dtype)
    R, C = -(-N // rw), -(-N // bc)
    buf = (ctypes.c_ubyte * (R * C))()
    st = load().fa_tile_map(N, d, in_dtype, mask_kind, window, ctypes.cast(buf, ctypes.c_void_p))
    if st != FA_OK:
        raise FaError(st, "fa_tile_map")
    flat = bytes(buf)
    return [list(flat[r * C:(r + 1) * C]) for r in range(R)]


def fa_fwd_schedule(B: int, H: int, N: int, d: int, in_dtype: int, mask_kind: int,
                    compute_units: int, H_kv: int = None, window: int = 0):
    """Forward work order: a list with one entry per workgroup, each the
    list of (batch*head, row tile) pairs it takes, in order."""
    G, R = ctypes.c_int(0), ctypes.c_int(0)
    lib = load()
    H_kv = H if H_kv is None else H_kv
    st = lib.fa_fwd_schedule(B, H, H_kv, N, d, in_dtype, mask_kind, window, compute_units,
                             ctypes.byref(G), ctypes.byref(R), None, 0)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_schedule")
    n = 2 * G.value * R.value
    buf = (ctypes.c_int * n)()
    st = lib.fa_fwd_schedule(B, H, H_kv, N, d, in_dtype, mask_kind, window, compute_units,
                             ctypes.byref(G), ctypes.byref(R), ctypes.cast(buf, ctypes.c_void_p), n)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_schedule")
    flat = list(buf)
    out = []
    for g in range(G.value):
        row = flat[2 * g * R.value:2 * (g + 1) * R.value]
        out.append([(row[2 * k], row[2 * k + 1]) for k in range(R.value) if row[2 * k] >= 0])
    return out


def fa_status_string(status: int) -> str:
    return load().fa_status_string(status).decode()


def fa_last_error() -> str:
    return load().fa_last_error().decode()


def fa_probe_mfma(which, a, b, d, stream) -> int:
    return load().fa_probe_mfma(which, a, b, d, stream)


def fa_mfma_ceiling(n_blocks, iters, clocks, sink, stream) -> int:
    return load().fa_mfma_ceiling(n_blocks, iters, clocks, sink, stream)


# ---- torch convenience --------------------------------------------------------
def _dtype_code(t):
    import torch
    codes = {torch.float32: FA_DTYPE_F32, torch.float16: FA_DTYPE_F16,
             torch.bfloat16: FA_DTYPE_BF16}
    if t not in codes:
        raise TypeError("unsupported dtype %s" % t)
    return codes[t]


def attention(q, k, v, scale=None, mask: str = "none", window: int = 0,
              out_dtype=None, record_tiles=None):
    """o, lse = softmax(scale q k^T + mask) v for device tensors q [B, H, N, d]
    and k, v [B, H_kv, N, d]; H_kv = H is plain multi-head attention, a
    smaller H_kv (dividing H) lets consecutive groups of H / H_kv query heads
    share one key/value head (``fa_fwd_gqa``).

    ``out_dtype`` is the input dtype (default) or torch.float32.  ``lse`` is
    float32 [B, H, N].  ``record_tiles``: optional zero-filled uint8 device
    tensor that receives the kernel's tile decisions (see fa.h; H_kv = H only).
    """
    import torch
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, H, N, d] and k, v [B, H_kv, N, d]")
    if (k.shape[0], k.shape[2], k.shape[3]) != (q.shape[0], q.shape[2], q.shape[3]):
        raise ValueError("k, v must match q in B, N and d")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous [B, H, N, d]")
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if H_kv < 1 or H % H_kv:
        raise ValueError("the key/value head count %d must divide H = %d" % (H_kv, H))
    if record_tiles is not None and H_kv != H:
        raise ValueError("record_tiles needs H_kv = H")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    o = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr())
    rest = (N, d, float(scale), MASKS[mask], int(window), _dtype_code(q.dtype),
            _dtype_code(out_dtype))
    with torch.cuda.device(q.device):
        if record_tiles is not None:
            st = fa_fwd_record_tiles(*ptrs, B, H, *rest, record_tiles.data_ptr(), stream)
        elif H_kv != H:
            st = fa_fwd_gqa(*ptrs, B, H, H_kv, *rest, stream)
        else:
            st = fa_fwd(*ptrs, B, H, *rest, stream)
    if st != FA_OK:
        raise FaError(st, "fa_fwd")
    return o, lse


def attention_fp8(q, k, v, scale=None, v_scale: float = 1.0, mask: str = "none",
                  window: int = 0, out_dtype=None):
    """o, lse of attention for E4M3 device tensors (torch.float8_e4m3fn, or
    uint8 holding E4M3 codes) q [B, H, N, d] and k, v [B, H_kv, N, d]:
    o = v_scale softmax(scale q k^T + mask) v with every code taken at its
    value (``fa_fwd_fp8``).  ``out_dtype``: torch.bfloat16 (default),
    torch.float16 or torch.float32; lse is float32 [B, H, N]."""
    import torch
    allowed = (torch.float8_e4m3fn, torch.uint8)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, H, N, d] and k, v [B, H_kv, N, d]")
    if (k.shape[0], k.shape[2], k.shape[3]) != (q.shape[0], q.shape[2], q.shape[3]):
        raise ValueError("k, v must match q in B, N and d")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if not all(t.dtype in allowed for t in (q, k, v)):
        raise ValueError("q, k, v must be float8_e4m3fn (or uint8 E4M3 codes)")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if H_kv < 1 or H % H_kv:
        raise ValueError("the key/value head count %d must divide H = %d" % (H_kv, H))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    o = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        B, H, H_kv, N, d, float(scale), float(v_scale), MASKS[mask], int(window),
                        _dtype_code(out_dtype), stream)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_fp8")
    return o, lse


def attention_bwd(q, k, v, o, lse, dout, scale=None, mask: str = "none", window: int = 0):
    """dq, dk, dv of attention for device tensors (f16/bf16): q, o, dout
    [B, H, N, d], k, v [B, H_kv, N, d] (H_kv dividing H; H_kv < H calls
    ``fa_bwd_gqa``), o and lse the forward call's outputs (o in the input
    dtype, lse float32 [B, H, N]), dout the gradient of the loss with
    respect to o.  Allocates dq, dk, dv and the float32 [B, H, N] workspace
    with torch and calls ``fa_bwd`` / ``fa_bwd_gqa`` on the current stream."""
    import torch
    if not (q.dim() == 4 and q.shape == o.shape == dout.shape and k.dim() == 4
            and k.shape == v.shape):
        raise ValueError("q, o, dout must be [B, H, N, d] and k, v [B, H_kv, N, d]")
    if (k.shape[0], k.shape[2], k.shape[3]) != (q.shape[0], q.shape[2], q.shape[3]):
        raise ValueError("k, v must match q in B, N and d")
    if lse.shape != q.shape[:3] or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, H, N]")
    ts = (q, k, v, o, lse, dout)
    if not all(t.is_cuda for t in ts):
        raise ValueError("all tensors must be device tensors")
    if not all(t.dtype == q.dtype for t in (k, v, o, dout)):
        raise ValueError("q, k, v, o, dout must share one dtype")
    if not all(t.is_contiguous() for t in ts):
        raise ValueError("all tensors must be contiguous")
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if H_kv < 1 or H % H_kv:
        raise ValueError("the key/value head count %d must divide H = %d" % (H_kv, H))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr())
    rest = (N, d, float(scale), MASKS[mask], int(window), _dtype_code(q.dtype), stream)
    with torch.cuda.device(q.device):
        if H_kv != H:
            st = fa_bwd_gqa(*ptrs, B, H, H_kv, *rest)
        else:
            st = fa_bwd(*ptrs, B, H, *rest)
    if st != FA_OK:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv


def attention_decode(q, k, v, scale=None, mask: str = "causal", window: int = 0, workspace=None):
    """o, lse for device tensors q [B, H, Nq, d] (the last Nq positions) and a
    key/value cache k, v [B, H_kv, Nk, d] (f16/bf16).  Allocates o, lse and,
    unless given (a uint8 device tensor), the workspace with torch, and calls
    ``fa_decode`` on the current stream."""
    import torch
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, H_kv, Nk, d]")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, Nq, d = q.shape
    H_kv, Nk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k, v must match q in B and d")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nbytes = fa_decode_workspace_bytes(B, H, H_kv, Nq, Nk, d)
    if nbytes < 0:
        raise FaError(FA_ERR_INVALID_ARG, "fa_decode_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    o = torch.empty((B, H, Nq, d), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       B, H, H_kv, Nq, Nk, d, float(scale), MASKS[mask], int(window),
                       _dtype_code(q.dtype), workspace.data_ptr(), workspace.numel(), stream)
    if st != FA_OK:
        raise FaError(st, "fa_decode")
    return o, lse
