"""The rocprofv3 summary tool (profsum) on small synthetic result databases:
counter traffic is scaled by what the same counter reads for a plain copy of
known size (the last three copy dispatches of the run), and the per-kernel
duration table averages each kernel's dispatches."""

import sqlite3

import pytest

from decode_megakernel_persistent_amd import profsum


def counter_db(path, counter, rows):
    c = sqlite3.connect(path)
    c.execute("create table counters_collection (kernel_name text, dispatch_id integer, counter_name text, "
              "value real)")
    for name, d, v in rows:
        # two entries per dispatch (as for a counter summed over instances)
        c.execute("insert into counters_collection values (?, ?, ?, ?)", (name, d, counter, v / 2))
        c.execute("insert into counters_collection values (?, ?, ?, ?)", (name, d, counter, v / 2))
    c.commit()
    c.close()


def test_traffic_scaled_by_plain_copies(tmp_path):
    mib = 64
    k = "void mk::mk_worker<1, false>(mk::StepArgs)"
    cp = "__amd_rocclr_copyBuffer"
    # FETCH_SIZE reads half the copied bytes on this part, WRITE_SIZE all of them
    fetch = [(cp, 1, 999.0), (k, 2, 1000.0), (k, 3, 1200.0), (cp, 4, mib * 512.0), (cp, 5, mib * 512.0),
             (cp, 6, mib * 512.0)]
    write = [(cp, 1, 5.0), (k, 2, 10.0), (k, 3, 30.0), (cp, 4, mib * 1024.0), (cp, 5, mib * 1024.0),
             (cp, 6, mib * 1024.0)]
    f, w = str(tmp_path / "f.db"), str(tmp_path / "w.db")
    counter_db(f, "FETCH_SIZE", fetch)
    counter_db(w, "WRITE_SIZE", write)
    out = profsum.traffic(f, w, "mk_worker", mib, 4400.0 * 1024, "cmd f", "cmd w")
    p = tmp_path / "t.txt"
    p.write_text(out)
    kv = profsum.read_kv(str(p))
    # kernel means 1100 KiB fetched (x2 calibration) and 20 KiB written (x1)
    assert float(kv["fetch_bytes_per_launch"]) == pytest.approx(2200 * 1024)
    assert float(kv["write_bytes_per_launch"]) == pytest.approx(20 * 1024)
    assert float(kv["traffic_bytes_per_launch"]) == pytest.approx(2220 * 1024)
    assert float(kv["traffic_over_algorithmic"]) == pytest.approx(2220 / 4400, abs=1e-4)  # printed to 4 places
    assert kv["command_fetch"] == "cmd f" and kv["kernel"] == "mk_worker"
    assert "source_hash" in kv


def test_stats_table(tmp_path):
    db = str(tmp_path / "k.db")
    c = sqlite3.connect(db)
    c.execute("create table kernels (name text, duration integer)")
    for d in (3000_000, 3100_000, 3200_000):
        c.execute("insert into kernels values (?, ?)", ("void mk::mk_worker<1, false>(mk::StepArgs)", d))
    c.execute("insert into kernels values (?, ?)", ("void mk::mk_dispatch(mk::StepArgs)", 3300_000))
    c.commit()
    c.close()
    out = profsum.stats(db, "the command")
    p = tmp_path / "s.txt"
    p.write_text(out)
    kv = profsum.read_kv(str(p))
    assert float(kv["mk_worker_avg_us"]) == pytest.approx(3100.0)
    assert int(kv["mk_worker_calls"]) == 3
    assert kv["command"] == "the command"
