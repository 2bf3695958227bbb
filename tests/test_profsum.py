"""Host checks of the rocprofv3 summary tool (profsum): trace table, calibrated traffic,
the source-hash guard bench.py relies on, and the counter summary. Synthetic inputs in
the layouts rocprofv3 writes (SQLite tables, counter_collection CSV)."""
import csv
import sqlite3

import pytest

from sparse_attention_autoregressive_amd import profsum


def _db(path, kernels=(), counters=()):
    c = sqlite3.connect(path)
    c.execute("create table kernels (name text, duration integer)")
    c.execute("create table counters_collection (kernel_name text, dispatch_id integer, counter_name text, value real)")
    c.executemany("insert into kernels values (?, ?)", kernels)
    c.executemany("insert into counters_collection values (?, ?, ?, ?)", counters)
    c.commit()
    c.close()
    return str(path)


def test_trace_lists_only_library_kernels(tmp_path):
    db = _db(tmp_path / "t.db", kernels=[("void lf::attn_bf16_kernel<128>(lf::AttnArgs)", 150_000),
                                        ("void lf::attn_bf16_kernel<128>(lf::AttnArgs)", 160_000),
                                        ("void at::native::copy_kernel(x)", 9_000)])
    out = profsum.trace(db, "T", "cmd")
    assert "| `void lf::attn_bf16_kernel<128>` | 2 | 155.00 | 155.00 | 150.00 |" in out
    assert "copy_kernel" not in out


def test_trace_splits_launch_shapes(tmp_path):
    c = sqlite3.connect(str(tmp_path / "g.db"))
    c.execute("create table kernels (name text, duration integer, grid_x integer, workgroup_x integer)")
    c.executemany("insert into kernels values (?, ?, ?, ?)",
                  [("lf::block_mean_kernel", 20_000, 256 * 900, 256), ("lf::block_mean_kernel", 22_000, 256 * 900, 256),
                   ("lf::block_mean_kernel", 6_000, 256 * 150, 256)])
    c.commit()
    c.close()
    out = profsum.trace(str(tmp_path / "g.db"), "T", "cmd")
    assert "| `lf::block_mean_kernel` | 900 | 2 | 21.00 | 21.00 | 20.00 |" in out
    assert "| `lf::block_mean_kernel` | 150 | 1 | 6.00 | 6.00 | 6.00 |" in out


def test_traffic_scales_each_counter_by_the_copy(tmp_path):
    # a 1 MiB calibration copy whose reads the counter reports twice over and whose
    # writes it reports exactly; the kernel's per-dispatch values are corrected alike
    fetch = _db(tmp_path / "f.db", counters=[("__amd_rocclr_copyBuffer", 1, "FETCH_SIZE", 2048.0),
                                             ("lf::attn_bf16_kernel", 2, "FETCH_SIZE", 600.0),
                                             ("lf::attn_bf16_kernel", 3, "FETCH_SIZE", 400.0),
                                             ("lf::attn_bf16_kernel", 4, "FETCH_SIZE", 500.0)])
    write = _db(tmp_path / "w.db", counters=[("__amd_rocclr_copyBuffer", 1, "WRITE_SIZE", 1024.0),
                                             ("lf::attn_bf16_kernel", 2, "WRITE_SIZE", 10.0)])
    out = profsum.traffic(fetch, write, "attn_bf16", 1, "wl", "cmd")
    kv = dict(line.split(": ", 1) for line in out.splitlines() if ": " in line and not line.startswith("#"))
    assert float(kv["fetch_factor"]) == pytest.approx(0.5)
    assert float(kv["write_factor"]) == pytest.approx(1.0)
    assert float(kv["fetch_kib_per_dispatch"]) == pytest.approx(500.0)          # median
    assert float(kv["traffic_bytes_per_dispatch"]) == pytest.approx((500.0 * 0.5 + 10.0) * 1024)
    assert kv["source_sha256"] == profsum.source_sha()


def test_traffic_summary_is_ignored_once_the_kernel_source_changes(tmp_path):
    good = tmp_path / "good.md"
    good.write_text(f"# x\nworkload: wl\nsource_sha256: {profsum.source_sha()}\ntraffic_bytes_per_dispatch: 1234\n")
    assert profsum.read_traffic(str(good)) == (1234.0, "wl")
    stale = tmp_path / "stale.md"
    stale.write_text("# x\nworkload: wl\nsource_sha256: 00\ntraffic_bytes_per_dispatch: 1234\n")
    assert profsum.read_traffic(str(stale)) is None
    assert profsum.read_traffic(str(tmp_path / "missing.md")) is None


def _csv(path, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))
    return str(path)


def test_counters_means_per_kernel_and_wave_cycle_split(tmp_path):
    attn, sel = "void lf::attn_bf16_kernel<128>(lf::AttnArgs)", "void lf::select_kernel<128, true, true>(x)"
    p1 = _csv(tmp_path / "a.csv", [(1, attn, "MfmaUtil", 30.0, 0, 150_000), (2, attn, "MfmaUtil", 40.0, 0, 160_000),
                                   (3, sel, "MfmaUtil", 0.0, 0, 9_000)])
    p2 = _csv(tmp_path / "b.csv", [(1, attn, "SQ_WAVE_CYCLES", 100.0, 0, 150_000),
                                   (1, attn, "SQ_WAIT_ANY", 25.0, 0, 150_000),
                                   (1, attn, "SQ_ACTIVE_INST_ANY", 40.0, 0, 150_000)])
    out = profsum.counters([p1, p2], "T", "rocprofv3 --pmc <set> -- x", ["MfmaUtil TD_BUSY_avr", None])
    assert "- `rocprofv3 --pmc MfmaUtil TD_BUSY_avr -- x`" in out
    assert "| attention | 2 | 35 | 100 | 25 | 40 |" in out
    assert "| selection | 1 | 0 | - | - | - |" in out
    assert "attention dispatch duration under counters: median 150.0 us" in out
    assert "- waiting on s_waitcnt (SQ_WAIT_ANY): 25.0%" in out
    assert "- issuing (SQ_ACTIVE_INST_ANY): 40.0%" in out


def test_counters_l2_hit_rate(tmp_path):
    attn = "void lf::attn_bf16_kernel<128>(lf::AttnArgs)"
    p = _csv(tmp_path / "c.csv", [(1, attn, "TCC_HIT_sum", 75.0, 0, 150_000), (1, attn, "TCC_MISS_sum", 25.0, 0, 150_000)])
    out = profsum.counters([p], "T", "x <set>")
    assert "- attention: 75.0% of 100 requests" in out
