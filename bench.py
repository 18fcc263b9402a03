"""Benchmark of the fused exact attention forward pass on one MI355X.

One step = one fa_fwd call over the whole workload (every step of the hot
path: Q/K/V tiles in, QK^T, mask and tile skipping, online softmax, P V, O
and lse out).  Default workload: B=1, H=32, N=16384, d=128, bf16, causal
(seeded N(0,1) synthetic inputs, resident in HBM before timing starts).

Prints ONE JSON line:
  value       whole-job TFLOP/s over the K timed steps (wall clock around the
              K launches, device synchronised on both sides); algorithmic
              FLOPs: 4*B*H*N^2*d, halved for causal, visible pairs for a
              sliding window
  roofline    the kernel's own average duration from HIP events recorded on
              the launch stream, against MI355X's dense bf16/fp16 matrix peak
              (2516.6 TFLOP/s: 256 CUs x 4096 FLOP/clk x 2.4 GHz); traffic =
              HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE
              (scaled by a plain copy's reading), when the recorded counters
              belong to the current kernel code (comments ignored), else null
  cpu_baseline the CPU oracle (fp64, OpenMP) timed on a bounded sample of the
              same workload's rows, in the same unit; context only

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       (NAME: one of seeded_inputs.BY_NAME, which includes the long-context
       shape with shared key/value heads, fa_fwd_gqa, and the E4M3 shapes,
       fa_fwd_fp8, timed against the 5033.2 TFLOP/s dense E4M3 peak)
       [--no-cpu-baseline] [--copy-calibration]
       python bench.py --n-sweep   (traffic-vs-N evidence, bf16 causal B=1 H=32 d=128)
       python bench.py --bwd       (backward pass, B=1 H=32 N=16384 d=128 bf16 causal;
                                    --workload picks another bf16 shape, e.g. the
                                    shared-head one, fa_bwd_gqa)
       python bench.py --decode    (decoding, B=8 H=32 H_kv=8 Nq=1 Nk=32768 d=128 bf16)
       python bench.py --hbm-reference   (torch sum / copy over 1 GiB, for context)
       python bench.py --record-traffic FETCH_CSV WRITE_CSV WORKLOAD "COMMAND"
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3, "e4m3": 5033.2}
METRIC = "attention fwd TFLOP/s + % bf16 MFMA peak (bf16 causal, N=16384, d=128)"
METRIC_FP8 = "attention fwd TFLOP/s + % E4M3 MFMA peak (e4m3 causal, N=16384, d=128)"
# Sources a forward workload's kernel is built from: its kernel file (8-bit
# inputs: fa_fwd8.hip, else fa_fwd.hip) and the shared ones.
SHARED_SOURCES = ["exact_io_aware_04_amd/csrc/fa_fwd_common.h", "exact_io_aware_04_amd/csrc/fa_device.h",
                  "exact_io_aware_04_amd/csrc/fa_kernels.h", "exact_io_aware_04_amd/csrc/tile_class.h",
                  "exact_io_aware_04_amd/csrc/fa_api.cpp"]
KERNEL_SOURCES = ["exact_io_aware_04_amd/csrc/fa_fwd.hip", "exact_io_aware_04_amd/csrc/fa_fwd8.hip"] + SHARED_SOURCES


def kernel_sources(w=None):
    """Source files of workload w's kernel (all forward sources for None)."""
    if w is None:
        return KERNEL_SOURCES
    main = "exact_io_aware_04_amd/csrc/fa_fwd8.hip" if w.dtype == "e4m3" else \
        "exact_io_aware_04_amd/csrc/fa_fwd.hip"
    return [main] + SHARED_SOURCES
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_fwd_traffic.json")


def code_text(src: str) -> str:
    """C/C++/HIP source with its comments removed and each run of whitespace
    collapsed to one newline (if the run holds one) or one space; string and
    character literals are kept as written.  Two sources with the same code
    text compile to the same program, so a comment edit does not void
    counters taken on the kernel."""
    out = []
    i, n = 0, len(src)
    pending = ""  # whitespace owed before the next token: "", " " or "\n"

    def emit(t):
        nonlocal pending
        if pending and out:
            out.append(pending)
        pending = ""
        out.append(t)

    def owe(ws):
        nonlocal pending
        if ws == "\n" or not pending:
            pending = ws

    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j  # the newline itself is whitespace
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            if j < 0:
                raise ValueError("unterminated block comment")
            owe("\n" if "\n" in src[i:j] else " ")
            i = j + 2
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            if j >= n:
                raise ValueError("unterminated literal")
            emit(src[i:j + 1])
            i = j + 1
        elif c.isspace():
            owe("\n" if c == "\n" else " ")
            i += 1
        else:
            emit(c)
            i += 1
    return "".join(out)


def kernel_source_hash(w=None) -> str:
    """SHA-256 of the code text (comments and layout ignored) of workload
    w's kernel sources (all forward sources for None)."""
    h = hashlib.sha256()
    for rel in kernel_sources(w):
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode("utf-8"))
        h.update(b"\0")
    return h.hexdigest()


def visible_pairs(N: int, mask: str, window: int) -> int:
    if mask == "none":
        return N * N
    if mask == "causal":
        return N * (N + 1) // 2
    w = min(window, N)
    return w * (w + 1) // 2 + (N - w) * w  # sum_i min(i + 1, w)


def step_flops(w) -> float:
    """Algorithmic FLOPs of one forward pass: 4*d per visible (query, key)
    pair for a sliding window; the conventional 4*B*H*N^2*d (halved when
    causal) otherwise."""
    if w.mask == "none":
        return 4.0 * w.B * w.H * w.N * w.N * w.d
    if w.mask == "causal":
        return 2.0 * w.B * w.H * w.N * w.N * w.d
    return 4.0 * w.B * w.H * w.d * visible_pairs(w.N, w.mask, w.window)


def algorithmic_bytes(w) -> int:
    """Q, K, V read once, O written once (input dtype; bf16 for E4M3
    inputs), lse written (fp32); K and V have kv_heads heads."""
    esz = {"f32": 4, "e4m3": 1}.get(w.dtype, 2)
    osz = 2 if w.dtype == "e4m3" else esz
    n = w.B * w.H * w.N
    n_kv = w.B * w.kv_heads * w.N
    return (n + 2 * n_kv) * w.d * esz + n * w.d * osz + 4 * n


def load_traffic(w):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on this workload with the current sources of its kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get("workloads", {}).get(w.name)
    if not ent or ent.get("kernel_src_sha256") != kernel_source_hash(w):
        return None
    return ent.get("hbm_bytes_per_launch")


def torch_index(rows):
    import torch
    return torch.from_numpy(rows)


def cpu_baseline(w, q, k, v, target_s: float = 12.0):
    """The oracle as it stands, timed on a bounded sample of the workload:
    whole heads (b=0, h=0, 1, ...) while they fit in about target_s seconds
    of CPU work, then evenly spaced rows of the next head; FLOPs counted as
    for the GPU (4*d per visible query-key pair)."""
    import numpy as np

    import oracle

    def flops_rows(rows):
        if w.mask == "none":
            cnt = np.full(len(rows), w.N)
        elif w.mask == "causal":
            cnt = rows + 1
        else:
            cnt = np.minimum(rows + 1, w.window)
        return 4.0 * w.d * float(cnt.sum())

    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    group = w.H // w.kv_heads

    def run(bh, rows):
        b, h = heads[bh]
        if w.dtype == "e4m3":  # the oracle decodes the codes first (timed)
            t0 = time.perf_counter()
            qq = oracle.decode_e4m3(q[b, h][torch_index(rows)])
            kk, vv = (oracle.decode_e4m3(t[b, h // group]) for t in (k, v))
            oracle.attention_rows(qq, rows, kk, vv, w.scale, w.mask, w.window)
            return time.perf_counter() - t0
        qq = q[b, h].double().numpy()
        kk, vv = (t[b, h // group].double().numpy() for t in (k, v))
        t0 = time.perf_counter()
        oracle.attention_rows(qq[rows], rows, kk, vv, w.scale, w.mask, w.window)
        return time.perf_counter() - t0

    probe = np.linspace(0, w.N - 1, 512).astype(np.int64)
    run(0, probe[:32])  # the first call pays thread start-up
    rate = flops_rows(probe) / max(run(0, probe), 1e-6)
    per_head = flops_rows(np.arange(w.N))
    budget = target_s * rate  # FLOPs to sample
    n_full = int(min(len(heads), budget // per_head))
    dt, fl, n_rows = 0.0, 0.0, 0
    for i in range(n_full):
        allr = np.arange(w.N)
        dt += run(i, allr)
        fl += per_head
        n_rows += w.N
    if n_full < len(heads):
        rem = int((budget - n_full * per_head) / (per_head / w.N))
        if rem >= 16:
            rows = np.linspace(0, w.N - 1, min(rem, w.N)).astype(np.int64)
            dt += run(n_full, rows)
            fl += flops_rows(rows)
            n_rows += len(rows)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "%d query rows of %s: %d whole heads plus evenly spaced rows of the "
                      "next (%.1f GFLOP, %.1f s)" % (n_rows, w.name, n_full, fl / 1e9, dt)}


def mfma_ceiling(torch, fa, n_blocks: int = 512, iters: int = 8000):
    """Sustained bf16 matrix-core throughput of this device (no memory
    traffic), and the shader clock it ran at: the measured ceiling next to
    the published peak."""
    import numpy as np

    dev = "cuda:0"
    clk = torch.zeros(n_blocks * 4, dtype=torch.int64, device=dev)
    sink = torch.empty(n_blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    args = (clk.data_ptr(), sink.data_ptr(), stream.cuda_stream)
    if fa.fa_mfma_ceiling(n_blocks, 200, *args) != fa.FA_OK:
        raise fa.FaError(fa.FA_ERR_HIP, "fa_mfma_ceiling")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    st = fa.fa_mfma_ceiling(n_blocks, iters, *args)
    e1.record(stream)
    torch.cuda.synchronize()
    if st != fa.FA_OK:
        raise fa.FaError(st, "fa_mfma_ceiling")
    ms = e0.elapsed_time(e1)
    c = clk.cpu().numpy().reshape(-1, 4).astype(np.float64)
    sclk = float(np.median((c[:, 1] - c[:, 0]) / (c[:, 3] - c[:, 2]))) * 0.1  # GHz
    flops = n_blocks * 4.0 * iters * 8 * 32768
    return {"tflops": round(flops / (ms * 1e-3) / 1e12, 1), "sclk_ghz": round(sclk, 3),
            "ms": round(ms, 3), "kind": "bf16 32x32x16 back-to-back, 8 chains/wave, 2 waves/SIMD"}


def copy_calibration(torch, nbytes: int = 1 << 30):
    """A plain device copy of known size, for scaling FETCH_SIZE/WRITE_SIZE."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 3}), flush=True)


def _pmc_rows(path):
    import csv
    rows = list(csv.DictReader(open(path)))
    per = {}
    for r in rows:
        key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
        per.setdefault(key, {}).setdefault(r["Counter_Name"], 0.0)
        per[key][r["Counter_Name"]] += float(r["Counter_Value"])
    return per


def record_traffic(fetch_csv: str, write_csv: str, workload: str, command: str):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch) of `bench.py --copy-calibration` into HBM bytes per launch of
    the attention kernel.  Each counter is scaled by bytes / reading of the
    plain copy of known size that the same run performs first."""
    import seeded_inputs as si

    out = {}
    for name, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        per = _pmc_rows(path)
        copies = [c[counter] for (d, k), c in sorted(per.items()) if "copyBuffer" in k]
        attn = [c[counter] for (d, k), c in sorted(per.items()) if "fa_fwd" in k]
        if not copies or not attn:
            raise SystemExit("no copy or attention dispatches in %s" % path)
        copy_kib = sorted(copies)[len(copies) // 2]
        scale = (1 << 30) / (copy_kib * 1024.0)
        kib = sum(attn) / len(attn)
        out[name] = {"kib_per_launch": kib, "copy_1GiB_reads_kib": copy_kib, "scale": scale,
                     "bytes_per_launch": kib * 1024.0 * scale, "launches": len(attn)}
    w = si.BY_NAME[workload]
    rec = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    rec.setdefault("workloads", {})
    rec.pop("kernel_src_sha256", None)
    hbm = out["fetch"]["bytes_per_launch"] + out["write"]["bytes_per_launch"]
    rec["workloads"][workload] = {
        "kernel_src_sha256": kernel_source_hash(w),
        "fetch": out["fetch"], "write": out["write"], "hbm_bytes_per_launch": round(hbm),
        "algorithmic_bytes": algorithmic_bytes(w), "ratio_to_algorithmic": hbm / algorithmic_bytes(w),
        "command": command}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec["workloads"][workload]))


SWEEP_N = (2048, 4096, 8192, 16384)


def sweep_traffic(fetch_csv: str, write_csv: str):
    """Traffic per N of an `--n-sweep` run under rocprofv3 --pmc FETCH_SIZE
    (then WRITE_SIZE; KiB per dispatch): the sweep launches the attention
    kernel three times per N, N in increasing order, so the k-th group of
    three attention dispatches is the k-th N.  FETCH_SIZE is scaled x2 and
    WRITE_SIZE x1, the factors a 1 GiB device copy calibrates."""
    rows = {}
    for name, path, counter, scale in (("fetch", fetch_csv, "FETCH_SIZE", 2.0),
                                       ("write", write_csv, "WRITE_SIZE", 1.0)):
        per = _pmc_rows(path)
        attn = [c[counter] for (d, k), c in sorted(per.items()) if "fa_fwd" in k]
        if len(attn) != 3 * len(SWEEP_N):
            raise SystemExit("%s: %d attention dispatches, expected %d" % (path, len(attn),
                                                                       3 * len(SWEEP_N)))
        for i, N in enumerate(SWEEP_N):
            three = sorted(attn[3 * i:3 * i + 3])
            rows.setdefault(N, {})[name] = three[1] * 1024.0 * scale  # median launch, bytes
    prev = None
    for N in SWEEP_N:
        qkv = 3 * 32 * N * 128 * 2
        tot = rows[N]["fetch"] + rows[N]["write"]
        slope = "" if prev is None else "%.2f" % (math.log2(tot / prev[1]) / math.log2(N / prev[0]))
        print(json.dumps({"N": N, "fetched_MB": round(rows[N]["fetch"] / 1e6, 1),
                          "x_qkv": round(rows[N]["fetch"] / qkv, 2),
                          "written_MB": round(rows[N]["write"] / 1e6, 1),
                          "total_MB": round(tot / 1e6, 1), "slope_vs_prev": slope}))
        prev = (N, tot)
    first, last = SWEEP_N[0], SWEEP_N[-1]
    t0 = rows[first]["fetch"] + rows[first]["write"]
    t1 = rows[last]["fetch"] + rows[last]["write"]
    print(json.dumps({"overall_slope": round(math.log2(t1 / t0) / math.log2(last / first), 3)}))


def n_sweep(torch, fa):
    """O(N) evidence: bf16 causal B=1 H=32 d=128 at N = 2048 .. 16384, seeded
    N(0,1) inputs, two warm-up launches and one timed launch per N, N in
    increasing order (sweep_traffic reads the counters of each N's three
    dispatches by that order)."""
    import numpy as np
    for N in SWEEP_N:
        rng = np.random.default_rng(2000 + N)
        shape = (1, 32, N, 128)
        q, k, v = (torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(torch.bfloat16).cuda()
                   for _ in range(3))
        o = torch.empty_like(q)
        lse = torch.empty((1, 32, N), dtype=torch.float32, device=q.device)
        stream = torch.cuda.current_stream()
        call = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), 1, 32, N, 128,
                128 ** -0.5, fa.FA_MASK_CAUSAL, 0, fa.FA_DTYPE_BF16, fa.FA_DTYPE_BF16, stream.cuda_stream)
        for _ in range(2):
            fa.fa_fwd(*call)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st = fa.fa_fwd(*call)
        e1.record(stream)
        torch.cuda.synchronize()
        if st != fa.FA_OK:
            raise fa.FaError(st, "fa_fwd")
        ms = e0.elapsed_time(e1)
        flops = 2.0 * 32 * N * N * 128
        print(json.dumps({"sweep": "bf16 causal B=1 H=32 d=128", "N": N, "kernel_ms": round(ms, 4),
                          "tflops": round(flops / ms / 1e9, 2)}), flush=True)


def bwd_bench(torch, fa, si, steps: int, warmup: int, w=None):
    """Backward pass (fa_bwd, or fa_bwd_gqa with shared key/value heads:
    delta, dq and dk/dv kernels) on a bf16 workload, by default the
    long-context shape B=1 H=32 N=16384 d=128 causal; seeded N(0,1) q, k, v
    and output gradient, o and lse from one forward call.  FLOPs: 2.5 x the
    forward's (five N x N x d products against two), the usual count; the
    kernels issue 3.5 x (S and dP are formed in both loop kernels)."""
    w = w or si.HEADLINE
    seed = 1010 if w is si.HEADLINE else w.seed + 100
    q, k, v, do = si.make_qkv_dout_shared(w.B, w.H, w.kv_heads, w.N, w.d, w.dtype, seed)
    dev = "cuda:0"
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.attention(qd, kd, vd, w.scale, w.mask, w.window)
    dq = torch.empty_like(qd)
    dk, dv = torch.empty_like(kd), torch.empty_like(vd)
    delta = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    ptrs = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
            dod.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr())
    rest = (w.N, w.d, float(w.scale), fa.MASKS[w.mask], int(w.window), fa.FA_DTYPE_BF16,
            stream.cuda_stream)
    if w.kv_heads == w.H:
        entry, call = fa.fa_bwd, ptrs + (w.B, w.H) + rest
    else:
        entry, call = fa.fa_bwd_gqa, ptrs + (w.B, w.H, w.kv_heads) + rest

    def step():
        st = entry(*call)
        if st != fa.FA_OK:
            raise fa.FaError(st, entry.__name__)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    flops = 2.5 * step_flops(w)
    avg = sum(ms) / len(ms)
    peak = PEAK_TFLOPS[w.dtype]
    print(json.dumps({
        "metric": "attention bwd TFLOP/s (bf16 causal, N=16384, d=128)",
        "value": round(flops * steps / wall / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(wall * 1e3 / steps, 4),
        "higher_is_better": True, "dtype": w.dtype, "data": "synthetic (seeded N(0,1), seed %d)" % seed,
        "config": {"workload": "bwd_" + w.name, "B": w.B, "H": w.H, "H_kv": w.kv_heads, "N": w.N, "d": w.d,
                   "mask": w.mask, "flops_per_step": flops, "flop_count": "2.5 x forward"},
        "roofline": {"bound": "mfma", "achieved": round(flops / (avg * 1e-3) / 1e12, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(flops / (avg * 1e-3) / 1e12 / peak, 4),
                     "call_avg_ms": round(avg, 4), "call_min_ms": round(min(ms), 4),
                     "note": "three kernels per call; per-kernel times from rocprofv3"}}),
        flush=True)


DECODE_SHAPE = dict(B=8, H=32, H_kv=8, Nq=1, Nk=32768, d=128)
HBM_PEAK_GBS = 8000.0


def decode_bytes(B, H, H_kv, Nq, Nk, d) -> int:
    """Algorithmic bytes of one decode call: the key/value cache read once,
    q read and o written (bf16), lse written (fp32)."""
    return 2 * B * H_kv * Nk * d * 2 + 2 * B * H * Nq * d * 2 + B * H * Nq * 4


def decode_bench(torch, fa, steps: int, warmup: int):
    """Decoding against a key/value cache (fa_decode: split and merge
    kernels): B=8 H=32 H_kv=8, one query per head at the end of a 32768-key
    bf16 cache, d=128, causal, seeded N(0,1) inputs resident in HBM.  Bound by
    HBM: reported in GB/s of algorithmic bytes against 8 TB/s."""
    import numpy as np
    c = DECODE_SHAPE
    rng = np.random.default_rng(1020)
    mk = lambda shape: torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(torch.bfloat16).cuda()
    q = mk((c["B"], c["H"], c["Nq"], c["d"]))
    k = mk((c["B"], c["H_kv"], c["Nk"], c["d"]))
    v = mk((c["B"], c["H_kv"], c["Nk"], c["d"]))
    o = torch.empty_like(q)
    lse = torch.empty((c["B"], c["H"], c["Nq"]), dtype=torch.float32, device=q.device)
    nb = fa.fa_decode_workspace_bytes(c["B"], c["H"], c["H_kv"], c["Nq"], c["Nk"], c["d"])
    ws = torch.empty(nb, dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream()
    scale = c["d"] ** -0.5
    call = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), c["B"], c["H"],
            c["H_kv"], c["Nq"], c["Nk"], c["d"], scale, fa.FA_MASK_CAUSAL, 0, fa.FA_DTYPE_BF16,
            ws.data_ptr(), nb, stream.cuda_stream)

    def step():
        st = fa.fa_decode(*call)
        if st != fa.FA_OK:
            raise fa.FaError(st, "fa_decode")

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    avg = sum(ms) / len(ms)
    nbytes = decode_bytes(**c)
    flops = 4.0 * c["B"] * c["H"] * c["Nq"] * c["Nk"] * c["d"]
    print(json.dumps({
        "metric": "attention decode GB/s (bf16, B=8 H=32 H_kv=8, 1 query, 32768 cached keys, d=128)",
        "value": round(nbytes * steps / wall / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(wall * 1e3 / steps, 4),
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic (seeded N(0,1), seed 1020)",
        "config": dict(workload="decode_bf16_b8_h32_hkv8_nq1_nk32768_d128", mask="causal",
                       bytes_per_step=nbytes, tflops=round(flops / (avg * 1e-3) / 1e12, 2), **c),
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (avg * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "call_avg_ms": round(avg, 4), "call_min_ms": round(min(ms), 4),
                     "note": "split and merge kernels per call; per-kernel times from rocprofv3"}}),
        flush=True)


def hbm_reference(torch):
    """Context for the HBM roofline: what torch's own kernels reach on this
    device -- a sum over 1 GiB of bf16 (reads 1 GiB) and a 1 GiB device copy
    (reads and writes 1 GiB) -- one JSON line each, ten timed calls."""
    x = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda").uniform_()
    y = torch.empty_like(x)
    for name, fn, nbytes in (("sum_bf16_1GiB", lambda: x.sum(), 1 << 30),
                             ("copy_1GiB", lambda: y.copy_(x), 2 << 30)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        print(json.dumps({"hbm_reference": name, "ms": round(ms, 4),
                          "GB_per_s": round(nbytes / ms / 1e6, 1)}), flush=True)


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--record-traffic":
        # --record-traffic FETCH_CSV WRITE_CSV WORKLOAD "COMMAND"
        record_traffic(*sys.argv[2:6])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--sweep-traffic":
        # --sweep-traffic FETCH_CSV WRITE_CSV (of two `--n-sweep` counter runs)
        sweep_traffic(*sys.argv[2:4])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--hbm-reference", action="store_true",
                    help="time torch's sum and copy over 1 GiB (context for the HBM roofline)")
    ap.add_argument("--decode", action="store_true",
                    help="time decoding (fa_decode) on B=8 H=32 H_kv=8 Nq=1 Nk=32768 d=128 bf16")
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward pass (fa_bwd) on B=1 H=32 N=16384 d=128 bf16 causal")
    ap.add_argument("--n-sweep", action="store_true",
                    help="bf16 causal B=1 H=32 d=128 at N = 2048..16384 (one timed launch each)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on exactly one GPU; --gpus %d is not supported (every "
              "(batch, head) slice is independent, so G GPUs would each run the same "
              "kernel on B*H/G heads)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_io_aware_04_amd as fa
    import seeded_inputs as si

    w = si.BY_NAME[args.workload] if args.workload else si.HEADLINE
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    fa.load()
    if args.copy_calibration:
        copy_calibration(torch)
    if args.n_sweep:
        n_sweep(torch, fa)
        return
    if args.bwd:
        if w.dtype != "bf16":
            print("bench.py --bwd times bf16 workloads", file=sys.stderr)
            sys.exit(2)
        bwd_bench(torch, fa, si, args.steps, args.warmup, w)
        return
    if args.decode:
        decode_bench(torch, fa, args.steps, args.warmup)
        return
    if args.hbm_reference:
        hbm_reference(torch)
        return

    q, k, v = si.make_workload(w)
    dev = "cuda:0"
    fp8 = w.dtype == "e4m3"
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty(qd.shape, dtype=torch.bfloat16 if fp8 else qd.dtype, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    ptrs = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr())
    if fp8:
        # E4M3 inputs, bf16 output, V factor 1
        entry = fa.fa_fwd_fp8
        call = ptrs + (w.B, w.H, w.kv_heads, w.N, w.d, float(w.scale), 1.0, fa.MASKS[w.mask],
                       int(w.window), fa.FA_DTYPE_BF16, stream.cuda_stream)
    else:
        dcode = {"f32": fa.FA_DTYPE_F32, "f16": fa.FA_DTYPE_F16, "bf16": fa.FA_DTYPE_BF16}[w.dtype]
        rest = (w.N, w.d, float(w.scale), fa.MASKS[w.mask], int(w.window), dcode, dcode,
                stream.cuda_stream)
        if w.kv_heads == w.H:
            entry, call = fa.fa_fwd, ptrs + (w.B, w.H) + rest
        else:
            entry, call = fa.fa_fwd_gqa, ptrs + (w.B, w.H, w.kv_heads) + rest

    def step():
        st = entry(*call)
        if st != fa.FA_OK:
            raise fa.FaError(st, entry.__name__)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps, device synchronised on both sides; one event
    # pair per launch on the launch stream gives the kernel's own duration
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [e0.elapsed_time(e1) for e0, e1 in ev]

    flops = step_flops(w)
    ms_per_step = wall * 1e3 / args.steps
    value = flops * args.steps / wall / 1e12
    avg_kern_ms = sum(kern_ms) / len(kern_ms)
    achieved = flops / (avg_kern_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    res = {
        "metric": METRIC_FP8 if fp8 else METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V%s, seed %d)" % (
            " cast to E4M3, bf16 output" if fp8 else "", w.seed),
        "config": {"workload": w.name, "B": w.B, "H": w.H, "H_kv": w.kv_heads, "N": w.N, "d": w.d,
                   "mask": w.mask, "window": w.window, "scale": w.scale,
                   "flops_per_step": flops, "pct_of_peak": round(100 * value / peak, 2),
                   "inputs_sha256": {"q": si.sha256(q), "k": si.sha256(k), "v": si.sha256(v)}},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": load_traffic(w),
                     "kernel_avg_ms": round(avg_kern_ms, 4),
                     "kernel_min_ms": round(min(kern_ms), 4),
                     "algorithmic_bytes": algorithmic_bytes(w)},
    }
    if w.dtype in ("bf16", "f16"):
        ceil = mfma_ceiling(torch, fa)
        res["roofline"]["measured_ceiling"] = ceil
        res["roofline"]["frac_of_measured_ceiling"] = round(achieved / ceil["tflops"], 4)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, q, k, v)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
