"""Host logic of bench.py, on the CPU: the one-GPU rule, the algorithmic FLOP and
byte counts its rates are computed from, the gate that reports HBM traffic only when
the committed counter summary was taken on the current kernel source, and the spread
statistics.  The expected counts are the ones stated for each workload from the
page's shapes (Wan-1.3B, VideoMLA Table 4 and App. D): 2*(2*d_c + d_rope) FLOP per
(query, key, head) of attention; x, both down-projection weights and the new ring
rows once for the cache write."""
import os
import shutil
import subprocess
import sys

import pytest

import bench
import workload as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("argv,needle", [(["--gpus", "2"], "one GPU only"),
                                         (["--gpus", "8"], "one GPU only"),
                                         (["--layers", "0"], "--layers must be >= 1")])
def test_bench_refuses_before_touching_a_gpu(argv, needle):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       capture_output=True, text=True, timeout=60, cwd=ROOT)
    assert r.returncode == 2 and needle in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name,tflop", [
    ("wan1.3b-w21", 1.5307),            # C1
    ("wan1.3b-w6-t240", 0.437), ("wan1.3b-w12-t240", 0.875), ("wan1.3b-w21-t240", 1.531),
    ("wan1.3b-w42-t240", 3.061), ("wan1.3b-w21-t240-q1", 0.510),   # C3
    ("wan1.3b-w21-dc128-dr32", 1.060), ("wan1.3b-w21-dc256-dr32", 2.002),
    ("wan1.3b-w21-dc192-dr64", 1.649),  # C4
])
def test_attention_flops(name, tflop):
    s = W.shape_by_name(name)
    assert bench.attention_flops(s) / 1e12 == pytest.approx(tflop, abs=6e-4)
    # the definition written out: every chunk token against the whole window
    assert bench.attention_flops(s) == 2 * s.chunk_tokens * s.window_tokens * s.n_heads * (
        2 * s.d_c + s.d_rope)


def test_step_and_cache_write_counts_at_wan13b():
    s = W.shape_by_name("wan1.3b-w21")
    f = bench.step_flops(s)
    assert f["total"] / 1e12 == pytest.approx(1.583, abs=5e-4)
    assert f["attention"] == bench.attention_flops(s)
    assert f["write"] / 1e9 == pytest.approx(3.22, abs=5e-3)
    assert f["out"] / 1e9 == pytest.approx(22.08, abs=5e-3)
    assert f["vup"] / 1e9 == pytest.approx(2.76, abs=5e-3)
    assert bench.cache_write_bytes(s) == 2 * (4680 * 1536 + 224 * 1536 + 4680 * 224)
    assert bench.cache_write_bytes(s) / 1e6 == pytest.approx(17.16, abs=5e-3)
    # a batch scales every count
    s3 = s.with_(batch=3)
    assert bench.step_flops(s3)["total"] == 3 * f["total"]
    assert bench.cache_write_bytes(s3) - 3 * bench.cache_write_bytes(s) == -2 * 2 * 224 * 1536
    # 30 layers of C1: 47.5 TFLOP
    assert 30 * f["total"] / 1e12 == pytest.approx(47.49, abs=0.01)


def test_causal_clip_counts_only_the_attended_pairs():
    s = W.shape_by_name("wan1.3b-clip21-causal3")
    tpf, blocks = s.tokens_per_frame, s.chunk_frames // s.causal_frames
    block = s.causal_frames * tpf
    pairs = sum(block * (k + 1) * block for k in range(blocks))   # block k sees blocks 0..k
    assert bench.attention_flops(s) == 2 * pairs * s.n_heads * (2 * s.d_c + s.d_rope)
    assert bench.attention_flops(s) / 1e12 == pytest.approx(6.12, abs=0.01)


def test_traffic_is_reported_only_for_the_profiled_source(tmp_path, monkeypatch):
    """The committed counter summaries carry the hash of the kernel source they were
    taken on; bench.py reports their traffic only while that source is unchanged."""
    import json
    csrc = os.path.join(ROOT, "latent_kv_attention_down_amd", "csrc")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    for src, summary in (("attention.hip", "latent_attention_wan1.3b_w21_traffic.json"),
                         ("cache_write.hip", "cache_write_wan1.3b_w21_traffic.json")):
        d = json.load(open(os.path.join(ROOT, "profiles", summary)))
        assert d["hbm_bytes_per_launch"] > 0 and "kernel_source_sha256_16" in d
        d["kernel_source_sha256_16"] = bench.source_hash(os.path.join(csrc, src))
        json.dump(d, open(tmp_path / "profiles" / summary, "w"))
        assert bench.traffic_from_profiles(os.path.join(csrc, src), summary) == \
            d["hbm_bytes_per_launch"]
        changed = tmp_path / src
        shutil.copy(os.path.join(csrc, src), changed)
        with open(changed, "a") as f:
            f.write("\n// edited\n")
        assert bench.traffic_from_profiles(str(changed), summary) is None
    assert bench.traffic_from_profiles(os.path.join(csrc, "attention.hip"), "missing.json") is None


def test_spread():
    assert bench.spread([4.0, 1.0, 3.0, 2.0, 5.0]) == {"mean": 3.0, "median": 3.0, "p10": 1.0,
                                                        "p90": 5.0}
    assert bench.spread([2.5]) == {"mean": 2.5, "median": 2.5, "p10": 2.5, "p90": 2.5}
