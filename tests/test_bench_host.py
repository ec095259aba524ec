"""CPU-only checks of bench.py's host logic: it refuses more than one GPU
before touching a device, its algorithmic byte/flop counts match the
definitions written out here, and the HBM-traffic record is reported only for
the kernel sources it was measured on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_algorithmic_work_decode_8x7b():
    cfg = dict(T=32, d=4096, ffn=14336, E=8, k=2, dtype="bf16")
    counts = [8, 7, 9, 8, 5, 6, 9, 12]
    layer_b, layer_f, gu_b, gu_f = bench.algorithmic_work(cfg, counts)
    d, F, T, A = 4096, 14336, 32, 64
    # every expert is active: 3 matrices of d*F bf16 each, x read, out written, router fp32
    assert layer_b == 8 * 3 * d * F * 2 + T * d * 2 + T * d * 2 + 8 * d * 4
    assert layer_f == 2 * A * 3 * d * F + 2 * T * 8 * d
    assert gu_b == 8 * 2 * d * F * 2 + T * d * 2 + A * F * 2
    assert gu_f == 2 * A * 2 * d * F
    # an idle expert's weights are not read
    assert bench.algorithmic_work(cfg, counts[:7] + [0])[2] == gu_b - 2 * d * F * 2


def test_traffic_record_is_tied_to_the_kernel_sources(tmp_path, monkeypatch):
    rec = {"ffn_sources_sha256": bench.ffn_sources_sha(),
           "workloads": {"decode_8x7b": {"hbm_bytes_per_launch": 123}}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.traffic_entry("decode_8x7b") == 123
    assert bench.traffic_entry("prefill_8x7b") is None
    rec["ffn_sources_sha256"] = "0" * 64
    path.write_text(json.dumps(rec))
    assert bench.traffic_entry("decode_8x7b") is None


def test_committed_traffic_record_is_current():
    """profiles/traffic.json was measured on the kernel sources as they are."""
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec.get("ffn_sources_sha256") != bench.ffn_sources_sha():
        pytest.skip("gate/up kernel sources changed since the counters were taken")
    assert rec["workloads"], "no workload recorded"
    for key, ent in rec["workloads"].items():
        assert ent["hbm_bytes_per_launch"] == ent["fetch_bytes"] + ent["write_bytes"], key
        if "down" in ent:
            d = ent["down"]
            assert d["hbm_bytes_per_launch"] == d["fetch_bytes"] + d["write_bytes"], key
    # the decode line's layout (standard) has its record
    assert "decode_8x7b+standard" in rec["workloads"]


def test_routing_workload_pairs_share_their_inputs():
    """Each (decode, prefill) pair of the routing-setting workloads differs only
    in T, so one draw serves both: the decode batch's x is the first rows of
    the prefill batch's (the generator fills x row by row), weights equal."""
    import numpy as np

    import gen
    for dname, pname in bench.ROUTING_WORKLOADS:
        dc, pc = dict(gen.CONFIGS[dname]), dict(gen.CONFIGS[pname])
        assert dc.pop("T") < pc.pop("T")
        assert dc == pc
    small = dict(d=64, ffn=64, E=4, k=1, dtype=gen.BF16, seed=5)
    a, b = gen.make_inputs(T=32, **small), gen.make_inputs(T=96, **small)
    assert np.array_equal(a["x"], b["x"][:32])
    assert all(np.array_equal(a[n], b[n]) for n in ("router", "w1", "w3", "w2"))


def test_down_work():
    cfg = dict(T=4096, d=4096, ffn=14336, E=8, k=2, dtype="bf16")
    b, f = bench.down_work(cfg, [1024] * 8)
    assert f == 2 * 8192 * 14336 * 4096
    assert b == 8 * 4096 * 14336 * 2 + 8192 * 14336 * 2 + 8192 * 4096 * 4
