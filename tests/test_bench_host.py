"""Host-side parts of bench.py, on the CPU: the one-GPU guard, the traffic figure's link to
the kernel source it was measured on, and the oracle baseline record."""
import json
import os
import subprocess
import sys

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_device_work():
    for extra, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + extra, capture_output=True,
                           text=True, timeout=120, env=dict(os.environ, **env), cwd=ROOT)
        assert r.returncode == 2 and "one GPU" in r.stderr, (extra, env, r.stderr)
        assert r.stdout == ""                    # no JSON line


def test_traffic_is_reported_only_for_the_profiled_kernel_source(tmp_path, monkeypatch):
    src = bench.kernel_source_hash()
    assert len(src) == 16 and int(src, 16) >= 0
    committed = os.path.join(bench.PROFILES, "chunk_attention_wan1.3b_hbm_traffic.json")
    d = json.load(open(committed))
    if d["kernel_source_hash"] == src:           # counters taken on this very source
        assert bench.traffic_from_profile("wan1.3b", src) == d["hbm_bytes_per_launch"] > 0
    else:                                        # the kernel changed since: no figure
        assert bench.traffic_from_profile("wan1.3b", src) is None
    assert bench.traffic_from_profile("wan1.3b", d["kernel_source_hash"]) == d["hbm_bytes_per_launch"]
    assert bench.traffic_from_profile("wan1.3b", "0" * 16) is None          # another source: no figure
    assert bench.traffic_from_profile("no_such_workload", src) is None
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    (tmp_path / "chunk_attention_x_hbm_traffic.json").write_text(json.dumps({"kernel_source_hash": src}))
    assert bench.traffic_from_profile("x", src) is None                    # no byte count recorded


def test_cpu_baseline_record():
    w = synth.small_variant(synth.WORKLOADS["wan1.3b"], heads=2, frame_h=4, frame_w=6, frames_per_chunk=2,
                            window_chunks=2)
    r = bench.cpu_baseline(w, 0.01)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["value"] > 0 and r["cores"] >= 1
    assert r["seconds_per_chunk"] > 0 and "heads of one steady-state chunk" in r["sample"]
    assert abs(r["value"] * r["seconds_per_chunk"] - w.batch * w.tokens_per_chunk) < 1e-6 * r["value"]


def test_tiny_stream_schedule_and_oracle_time():
    w = synth.WORKLOADS["tiny_f32"]
    ops = []
    bench._tiny_schedule(w, lambda c: ops.append(("attend", c)), lambda c: ops.append(("append", c)),
                         lambda: ops.append(("refresh", None)))
    want = []
    for c in range(w.n_chunks):
        if c == 4:                                   # refresh every 4 chunks, none before chunk 0
            want.append(("refresh", None))
        want += [("attend", c), ("append", c)]
    assert ops == want
    assert bench.tiny_oracle(synth, reps=1) > 0
