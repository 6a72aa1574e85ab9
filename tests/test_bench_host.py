"""Host logic of bench.py (no GPU): the one-GPU guard, the HBM byte records written from
rocprofv3 counter databases, and the digest check that retires stale records."""
import json
import os
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_cluster_mean_splits_two_workloads_at_the_widest_gap():
    vals = [100.0, 101.0, 99.0, 150.0, 149.0, 151.0, 100.5]
    assert bench._cluster_mean(vals, 0) == pytest.approx((100 + 101 + 99 + 100.5) / 4)
    assert bench._cluster_mean(vals, 1) == pytest.approx(150.0)
    assert bench._cluster_mean(vals, None) == pytest.approx(sum(vals) / len(vals))
    # one cluster (gap below 1% of the largest value): both sides get the mean
    assert bench._cluster_mean([100.0, 100.2, 100.1], 1) == pytest.approx(100.1)


def _counter_db(path, counter, rows):
    """rows: (kernel name, value) or (kernel name, value, grid in threads)."""
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, grid_size integer, counter_name text, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?)",
                    [(r[0], r[2] if len(r) > 2 else 64, counter, r[1]) for r in rows])
    con.commit()
    con.close()


def test_write_traffic_from_counter_databases(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    # a 1 GiB copy that reports half its bytes on FETCH_SIZE and all of them on WRITE_SIZE
    fetch = [(copy, 524288.0), (copy, 524288.0), (copy, 8.0)]
    write = [(copy, 1048576.0), (copy, 1048576.0)]
    fwd_vals = {}
    for i, (key, src, kname, which) in enumerate(bench.TRAFFIC_KERNELS):
        base = {"fwd": 1000.0, "decode": 5000.0, "bwd": 7000.0}[src]
        grid = bench.TRAFFIC_GRID.get(key)
        # one forward kernel on several grids: each record takes only its own grid's dispatches (the
        # causal and unmasked launches share one grid and are told apart by their byte counts)
        if grid:
            fwd_vals[key] = base + 100.0 * i
            fetch.append((f"void attn::{kname}(args)", fwd_vals[key], grid))
            write.append((f"void attn::{kname}(args)", 10.0, grid))
        elif which is None:
            fetch.append((f"void attn::{kname}(args)", base))
            write.append((f"void attn::{kname}(args)", 10.0))
    # the two INT4 workloads share a kernel name: values 3000 (G=1) and 3500 (G=4)
    int4 = "void attn::decode_kernel<128, 3, 0, false>(args)"
    fetch += [(int4, 3000.0), (int4, 3001.0), (int4, 3500.0), (int4, 3499.0)]
    write += [(int4, 20.0), (int4, 20.0)]
    fdb, wdb, out = tmp_path / "f.db", tmp_path / "w.db", tmp_path / "traffic.json"
    _counter_db(fdb, "FETCH_SIZE", fetch)
    _counter_db(wdb, "WRITE_SIZE", write)
    bench.write_traffic(str(fdb), str(wdb), out_path=str(out))
    rec = json.loads(out.read_text())
    assert set(rec) == {k for k, *_ in bench.TRAFFIC_KERNELS}
    g1, g4 = rec["decode int4 g1 16x32768x32x128 s32"], rec["decode int4 g4 16x32768x32x128 s32"]
    assert g1["fetch_kib"] == pytest.approx(3000.5) and g4["fetch_kib"] == pytest.approx(3499.5)
    assert g1["fetch_scale"] == pytest.approx(2.0) and g1["write_scale"] == pytest.approx(1.0)
    fwd = rec["fwd_bf16 causal 2x2048x32x128"]
    assert fwd["source_sha256"] == bench.kernel_source_digest("fwd")
    for key, val in fwd_vals.items():
        assert rec[key]["fetch_kib"] == pytest.approx(val)
    for key in ("bwd dq causal 2x2048x32x128", "bwd dkdv causal 2x2048x32x128"):
        assert rec[key]["fetch_kib"] == pytest.approx(7000.0)
        assert rec[key]["source_sha256"] == bench.kernel_source_digest("bwd")
    # bytes per launch = FETCH x scale + WRITE x scale, in bytes
    assert bench.recorded_traffic("fwd_bf16 causal 2x2048x32x128", str(out)) == pytest.approx(
        (fwd_vals["fwd_bf16 causal 2x2048x32x128"] * 2.0 + 10.0) * 1024)


def test_stale_digest_retires_the_record(tmp_path):
    out = tmp_path / "traffic.json"
    out.write_text(json.dumps({"k": {"sources": "decode", "source_sha256": "0" * 64, "fetch_kib": 1.0,
                                     "fetch_scale": 2.0, "write_kib": 1.0, "write_scale": 1.0}}))
    assert bench.recorded_traffic("k", str(out)) is None
    rec = json.loads(out.read_text())
    rec["k"]["source_sha256"] = bench.kernel_source_digest("decode")
    out.write_text(json.dumps(rec))
    assert bench.recorded_traffic("k", str(out)) == pytest.approx(3 * 1024)
