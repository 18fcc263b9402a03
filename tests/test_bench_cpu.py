"""Host logic of bench.py, without a GPU: the work and byte counts it divides
by, the kernel-code fingerprint that ties recorded HBM counters to a kernel,
and the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

import bench
import seeded_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def brute_visible_pairs(N, mask, window):
    n = 0
    for i in range(N):
        for j in range(N):
            if mask == "none":
                n += 1
            elif mask == "causal":
                n += j <= i
            else:
                n += i - window < j <= i
    return n


@pytest.mark.parametrize("N", [1, 2, 5, 17, 40])
def test_visible_pairs_against_brute_force(N):
    assert bench.visible_pairs(N, "none", 0) == brute_visible_pairs(N, "none", 0)
    assert bench.visible_pairs(N, "causal", 0) == brute_visible_pairs(N, "causal", 0)
    for w in (1, 2, 3, N - 1, N, N + 7):
        if w >= 1:
            assert bench.visible_pairs(N, "sliding", w) == brute_visible_pairs(N, "sliding", w), w


def test_flop_and_byte_counts_of_the_workloads():
    h = si.HEADLINE
    assert (h.B, h.H, h.N, h.d, h.mask) == (1, 32, 16384, 128, "causal")
    assert bench.step_flops(h) == 2.0 * 32 * 16384 ** 2 * 128 == 2199023255552
    # Q, K, V read and O written once in bf16, lse written in fp32
    assert bench.algorithmic_bytes(h) == 4 * 32 * 16384 * 128 * 2 + 4 * 32 * 16384 == 538968064
    for w in si.WORKLOADS:
        pairs = bench.visible_pairs(w.N, w.mask, w.window)
        if w.mask == "sliding":
            assert bench.step_flops(w) == 4.0 * w.B * w.H * w.d * pairs
        else:
            full = 4.0 * w.B * w.H * w.N * w.N * w.d
            assert bench.step_flops(w) == (full / 2 if w.mask == "causal" else full)


def test_code_text_drops_comments_and_layout_only():
    src = 'int a = 1; // one\n/* two\n three */  int b=2;\nconst char* s = "// kept /* too */";\n'
    t = bench.code_text(src)
    assert "one" not in t and "three" not in t
    assert '"// kept /* too */"' in t
    assert bench.code_text(src.replace("// one", "// a longer comment")) == t
    assert bench.code_text(src.replace("  int b", "\n\n   int b")) == t
    assert bench.code_text(src.replace("b=2", "b=3")) != t
    assert bench.code_text(src.replace("int b", "intb")) != t
    with pytest.raises(ValueError):
        bench.code_text("int a; /* open")


def test_kernel_fingerprint_follows_code_not_comments(tmp_path, monkeypatch):
    rel = bench.KERNEL_SOURCES[0]
    src = open(os.path.join(ROOT, rel), encoding="utf-8").read()
    for r in bench.KERNEL_SOURCES:
        p = tmp_path / r
        p.parent.mkdir(parents=True, exist_ok=True)
        p.write_text(open(os.path.join(ROOT, r), encoding="utf-8").read(), encoding="utf-8")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    h16, h8 = bench.kernel_source_hash(si.HEADLINE), bench.kernel_source_hash(si.FP8_WORKLOADS[0])
    assert len({h0, h16, h8}) == 3
    (tmp_path / rel).write_text("// a new comment line\n" + src.replace("\n", "\n\n", 3),
                                encoding="utf-8")
    assert bench.kernel_source_hash() == h0
    (tmp_path / rel).write_text(src.replace("#define FA_OPND_AHEAD 6", "#define FA_OPND_AHEAD 4"),
                                encoding="utf-8")
    assert bench.kernel_source_hash() != h0
    # a change to the 16-bit kernel voids its workloads' records, not the 8-bit one's
    assert bench.kernel_source_hash(si.HEADLINE) != h16
    assert bench.kernel_source_hash(si.FP8_WORKLOADS[0]) == h8


def test_traffic_record_is_used_only_for_the_current_kernel(tmp_path, monkeypatch):
    w = si.HEADLINE
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.load_traffic(w) is None  # no record
    rec = {"workloads": {w.name: {"kernel_src_sha256": bench.kernel_source_hash(w),
                                  "hbm_bytes_per_launch": 123456789}}}
    f.write_text(json.dumps(rec))
    assert bench.load_traffic(w) == 123456789
    assert bench.load_traffic(si.WORKLOADS[0]) is None  # another workload
    rec["workloads"][w.name]["kernel_src_sha256"] = bench.kernel_source_hash(si.FP8_WORKLOADS[0])
    f.write_text(json.dumps(rec))
    assert bench.load_traffic(w) is None  # counters of another kernel


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr and r.stdout == ""


def test_sweep_traffic_groups_dispatches_by_order(tmp_path, capsys):
    """--sweep-traffic: the k-th group of three attention dispatches is the
    k-th N; other kernels in between are ignored; the median launch is used."""
    import json as _json

    def csv(path, counter, vals):
        lines = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
        d = 0
        for i, N in enumerate(bench.SWEEP_N):
            d += 1
            lines.append("%d,fill_kernel,%s,5" % (d, counter))
            for j in range(3):
                d += 1
                lines.append("%d,fa_fwd16_kernel<2; 128; false>,%s,%s" % (d, counter, vals(i, j)))
        path.write_text("\n".join(lines) + "\n")

    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    csv(f, "FETCH_SIZE", lambda i, j: 1000 * 4 ** i + j)   # median = 1000 * 4^i + 1
    csv(w, "WRITE_SIZE", lambda i, j: 100 * 2 ** i)
    bench.sweep_traffic(str(f), str(w))
    out = [_json.loads(l) for l in capsys.readouterr().out.splitlines()]
    assert [o["N"] for o in out[:-1]] == list(bench.SWEEP_N)
    assert out[0]["fetched_MB"] == round((1000 + 1) * 1024 * 2 / 1e6, 1)
    assert out[3]["written_MB"] == round(800 * 1024 / 1e6, 1)
    assert 1.8 < out[-1]["overall_slope"] < 2.0
