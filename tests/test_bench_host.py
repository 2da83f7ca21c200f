"""Host logic of bench.py, no GPU: the one-GPU refusal, the traffic records' staleness
rule, and the algorithmic byte and flop counts its roofline divides by (checked
against the sizes of the arrays the input generators actually produce)."""
import dataclasses
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import hy_inputs as hi  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_source_digest_ignores_comments_and_whitespace(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f(int x) { return x + 1; }\n")
    b.write_text("// a note\nint f(int x) {\n  /* block\n comment */ return x + 1;  // done\n}\n")
    c.write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_digest(str(a)) == bench.source_digest(str(b))
    assert bench.source_digest(str(a)) != bench.source_digest(str(c))


def test_traffic_records_go_stale_with_their_source(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("__global__ void k() {}\n")
    rec = {"bytes_per_launch": 123.0, "source": str(src), "source_sha256_16": bench.source_digest(str(src))}
    tf = tmp_path / "traffic.json"
    tf.write_text(json.dumps({"kern/work": rec}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    assert bench.traffic_for("kern/work", 1) == 123.0
    assert bench.traffic_for("kern/other", 1) is None
    src.write_text("__global__ void k() { int x = 0; }\n")  # the kernel changed since
    assert bench.traffic_for("kern/work", 1) is None


def test_committed_traffic_records_follow_their_sources():
    """A counter record is reported while its kernel source is the one the counters were
    taken on, and reported as absent (null) once that source has changed."""
    recs = json.load(open(bench.TRAFFIC_FILE))
    for key, rec in recs.items():
        current = bench.source_digest(os.path.join(bench.ROOT, rec["source"])) == rec["source_sha256_16"]
        assert bench.traffic_for(key, 1) == (rec["bytes_per_launch"] if current else None), key


def _nbytes(arrays, keys):
    return sum(arrays[k].nbytes for k in keys)


@pytest.mark.parametrize("fmt", ["bf16", "ternary", "fp8"])
def test_stream_bytes_equal_the_generated_arrays(fmt):
    """Per touched expert, the counted bytes are those of the arrays the generators make
    (small shape, so the arrays are cheap), and the layer adds router, x and output."""
    cfg = hi.LayerConfig("b", T=8, d=512, E=8, k=2, I=256, ternary=fmt == "ternary", fp8=fmt == "fp8")
    touched = 5
    w = bench.stream_work(cfg, touched)
    shared = hi.host_shared(cfg)
    if fmt == "bf16":
        ex = hi.host_expert(cfg, 0)
        gu = _nbytes(ex, ["gate", "up"])
        allw = _nbytes(ex, ["gate", "up", "down"])
        assert w["alg"] == (touched + 1) * gu
        experts = (touched + 1) * allw
    else:
        ex = hi.host_expert_ternary(cfg, 0) if fmt == "ternary" else hi.host_expert_fp8(cfg, 0)
        p = "q" if fmt == "ternary" else "f"
        s = "s" if fmt == "ternary" else "fs"
        gu = _nbytes(ex, [p + "gate", p + "up", s + "gate", s + "up"])
        allw = _nbytes(ex, [p + "gate", p + "up", p + "down", s + "gate", s + "up", s + "down"])
        assert w["alg"] == touched * gu + _nbytes(shared, ["gate", "up"])
        experts = touched * allw + _nbytes(shared, ["gate", "up", "down"])
    assert w["unit"] == gu
    x = hi.host_x(cfg)
    assert w["layer_bytes"] == experts + hi.host_router(cfg).nbytes + 2 * x.nbytes


def test_sherry_expert_bytes_at_full_size():
    """The Sherry layout (5 words per 128 weights, bf16 row scales) gives 5,918,720 bytes
    per routed expert of the d=6144, I=2048 layer (the scope table's figure)."""
    cfg = hi.CONFIGS["ternary"]
    one = bench.stream_work(cfg, 1)["layer_bytes"] - bench.stream_work(cfg, 0)["layer_bytes"]
    assert one == 5_918_720


def test_decode_layer_bytes_and_unit():
    cfg = hi.CONFIGS["decode"]
    w = bench.stream_work(cfg, 156)
    assert w["unit"] == 50_331_648 and w["key"] == "stream_gateup"
    assert w["layer_bytes"] == 157 * 3 * 2048 * 6144 * 2 + 256 * 6144 * 2 + 2 * 32 * 6144 * 2
    assert bench.stream_work(hi.CONFIGS["ternary"], 1)["key"] == "ternary_gateup"


def test_prefill_flops():
    cfg = hi.CONFIGS["prefill"]
    w = bench.gemm_work(cfg)
    assert w["rows"] == 8192 * 8 + 8192
    assert w["alg"] == w["rows"] * 50_331_648
    # router (2 T d E) + gate, up and down (2 d I each) per dispatched row
    assert w["layer_flop"] == 2 * 8192 * 6144 * 256 + w["rows"] * 3 * 2 * 6144 * 2048
    # a different expert format changes the kernel, not the flop count
    assert bench.gemm_work(dataclasses.replace(cfg, fp8=True))["alg"] == w["alg"]


def test_w8a8_blended_peak():
    # routed rows run on FP8 MFMAs (5.0 PFLOP/s), shared rows on bf16 ones (2.5): with
    # 8 routed rows per shared row the stage's peak is 9 / (8 / 5.0 + 1 / 2.5) PFLOP/s
    cfg = hi.CONFIGS["fp8_w8a8_prefill"]
    w = bench.gemm_work(cfg)
    assert w["alg"] == bench.gemm_work(hi.CONFIGS["prefill"])["alg"]
    assert abs(w["peak"] - 9 / (8 / 5.0e15 + 1 / 2.5e15)) < 1e3
    assert bench.PEAK_BF16 < w["layer_peak"] < bench.PEAK_FP8
    assert bench.gemm_work(hi.CONFIGS["prefill"])["peak"] == bench.PEAK_BF16
