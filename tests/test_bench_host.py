"""Host-side pieces of bench.py that the reported numbers rest on (CPU only).

* The algorithmic bytes of a decode call are the sum the roofline divides by: every cached token's K and V
  row per head, the q and out rows, the block-table entries a decode reads and the lengths.  Checked here
  against a count made independently from the block tables themselves, on every configuration.
* An HBM-traffic summary is used only for the kernel, workload and split it was measured on.
* One GPU only: more is refused with a message.
"""
import json
import os
import subprocess
import sys

import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("cfg_id", sorted(W.CONFIGS))
def test_algorithmic_bytes_count_every_row_read(cfg_id):
    meta = W.make_metadata(cfg_id)
    cfg = meta.cfg
    es = 4 if cfg.dtype == "f32" else 2
    kv, tables = 0, 0
    for i, L in enumerate(meta.context_lens.tolist()):
        ids = meta.block_tables[i][meta.block_tables[i] >= 0]          # the blocks the sequence holds
        assert len(ids) * cfg.block_size >= L > (len(ids) - 1) * cfg.block_size
        tables += 4 * len(ids)
        for j in range(len(ids)):                                       # tokens of block j, K and V, all heads
            kv += min(cfg.block_size, L - j * cfg.block_size) * cfg.num_heads * cfg.head_dim * 2 * es
    B = len(meta.context_lens)
    want = kv + 2 * B * cfg.num_heads * cfg.head_dim * es + tables + 4 * B
    got = bench.algorithmic_bytes(meta)
    assert got["kv"] == kv
    assert got["decode"] == want
    assert got["step"] == want + 2 * B * cfg.num_heads * cfg.head_dim * es * 2 + 8 * B


def test_traffic_summary_applies_only_to_its_kernel(tmp_path, monkeypatch):
    rec = {"workload": "llama2_13b_layer_b64_h40_d128_ctx128-2048_bf16", "partition_size": 0,
           "kernel_sha256": bench.kernel_fingerprint(), "bytes_per_launch": 1545509970,
           "fetch_scale": 1.99998, "write_scale": 1.0}
    f = tmp_path / "traffic.md"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    f.write_text("# summary\n\ntraffic-json: " + json.dumps(rec) + "\n")
    assert bench.measured_traffic(rec["workload"], 0) == rec
    assert bench.measured_traffic(rec["workload"], 512) is None          # another partition size
    assert bench.measured_traffic("another workload", 0) is None
    # a summary taken on another version of the kernel is not used
    f.write_text("traffic-json: " + json.dumps(dict(rec, kernel_sha256="0" * 64)) + "\n")
    assert bench.measured_traffic(rec["workload"], 0) is None


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in (res.stdout + res.stderr)


def test_cpu_oracle_steps_runs_whole_oracle_steps():
    """The CPU baseline of the secondary workloads: whole oracle steps (block copies, write, decode) on a tiny
    batch, its rate in the caller's byte count, every row with a context counted once per step."""
    import numpy as np
    rng = np.random.default_rng(7)
    H, D, bs, NB = 2, 64, 16, 12
    k0 = rng.standard_normal((NB, H, bs, D)).astype(np.float32)
    v0 = rng.standard_normal((NB, H, bs, D)).astype(np.float32)
    tables = np.array([[0, 1, -1], [2, -1, -1], [-1, -1, -1]], dtype=np.int32)
    lens = np.array([20, 5, 0], dtype=np.int32)                  # the empty row is skipped
    q = rng.standard_normal((3, H, D)).astype(np.float32)
    kn = rng.standard_normal((3, H, D)).astype(np.float32)
    vn = rng.standard_normal((3, H, D)).astype(np.float32)
    slots = np.array([1 * bs + 3, 2 * bs + 4, -1], dtype=np.int64)
    r = bench.cpu_oracle_steps(q, k0, v0, kn, vn, tables, lens, slots, 0.125, bs, "f32", step_bytes=10**6,
                               copies=[[2, 5]], budget_s=0.2, what="a test step")
    steps = int(r["sample"].split(" x ")[0])
    assert steps >= 1 and r["kind"] == "oracle" and r["unit"] == "GB/s" and r["cores"] >= 1
    assert r["tokens_heads_per_s"] > 0 and r["value"] > 0
    assert "2 rows each" in r["sample"] and "a test step" in r["sample"]
