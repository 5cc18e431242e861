"""bench.py's counter record on synthetic rocprofv3 counter files: kernel
instances keyed with their template arguments (the two passes of a shared
decode stay apart), the cascade merge counted with the decode call, other
kernels listed apart, bytes scaled by the copy calibration."""
import argparse
import csv
import os

import bench


def _write(folder, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, counter, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def _k(inner):
    return f"void pa::(anonymous namespace)::{inner}(pa::DecodeArgs, int)"


def test_counters_summary(tmp_path):
    tail = _k("decode_valu_kernel<pa::BF16, 128, 2, false, 1>")
    pre = _k("decode_mfma_kernel<pa::BF16, 128, false, 2>")
    merge = _k("cascade_merge_kernel<pa::BF16>")
    write = _k("reshape_and_cache_small_kernel<2>")
    copy = "void at::native::elementwise_kernel<copy_something>(int)"
    f, w, cf, cw = (str(tmp_path / x) for x in ("f", "w", "cf", "cw"))
    _write(f, [(tail, "FETCH_SIZE", 100), (tail, "FETCH_SIZE", 300), (tail, "FETCH_SIZE", 200),
               (pre, "FETCH_SIZE", 50), (merge, "FETCH_SIZE", 10), (write, "FETCH_SIZE", 7)])
    _write(w, [(tail, "WRITE_SIZE", 4), (pre, "WRITE_SIZE", 6), (merge, "WRITE_SIZE", 8),
               (write, "WRITE_SIZE", 9)])
    _write(cf, [(copy, "FETCH_SIZE", 2 * 1024 * 1024)])   # counter reads 2x the copied KiB
    _write(cw, [(copy, "WRITE_SIZE", 1024 * 1024 // 2)])  # ... and half for writes
    args = argparse.Namespace(counters_summary=[f, w, cf, cw], workload="llama13b_prefix_share",
                              partition=None)
    rec = bench.counters_summary(args)
    assert rec["fetch_scale"] == 0.5 and rec["write_scale"] == 2.0
    ks = rec["kernels"]
    assert set(ks) == {"decode_valu_kernel<pa::BF16, 128, 2, false, 1>",
                       "decode_mfma_kernel<pa::BF16, 128, false, 2>",
                       "cascade_merge_kernel<pa::BF16>"}
    assert ks["decode_valu_kernel<pa::BF16, 128, 2, false, 1>"] == {"fetch_bytes": 200 * 512,
                                                                   "write_bytes": 4 * 2048}
    assert set(rec["other_kernels"]) == {"reshape_and_cache_small_kernel<2>"}
    want = (200 + 50 + 10) * 512 + (4 + 6 + 8) * 2048
    assert rec["bytes_per_call"] == want


def test_prefill_roofline_picks_the_binding_roof():
    """The roof of a chunked-prefill call is the longer of its matrix-core
    time and its HBM time; the ridge is 2.5 PFLOP/s over 8 TB/s = 312.5
    flop per byte.  The 66B chunk writers (651.6 GFLOP over 2.62 GB of K/V,
    249 flop per byte) sit below it, so HBM binds."""
    flops, kv, sec = 651.6e9, 2.62e9, 0.86e-3
    r = bench.prefill_roofline(flops, kv, sec, 2500.0)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["achieved"] - kv / sec / 1e9) < 0.01
    assert abs(r["frac"] - kv / sec / 8e12) < 1e-4
    # ten times the flops on the same bytes: above the ridge, the matrix cores bind
    r = bench.prefill_roofline(10 * flops, kv, sec, 2500.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert abs(r["frac"] - 10 * flops / sec / 2.5e15) < 1e-4
    # exactly at the ridge both times are equal: reported against the matrix peak
    assert bench.prefill_roofline(312.5 * kv, kv, sec, 2500.0)["bound"] == "mfma"


def test_stored_records_follow_the_kernel_sources(tmp_path, monkeypatch):
    """The traffic and MFMA records under profiles/ were taken with the
    kernel sources as committed (bench.py reports them only then), and a
    record of other sources is ignored."""
    for wl in ("opt13b_decode", "gqa_long", "llama13b_prefix_share", "opt66b_sweep"):
        got = bench.stored_traffic(wl, None)
        assert isinstance(got, int) and got > 0, wl
    assert bench.stored_mfma("gqa_long", None) > 0
    rec = {"workload": "opt13b_decode", "partition": None, "sources_sha256": "0" * 16,
           "bytes_per_call": 1}
    (tmp_path / "old.md").write_text(bench.RECORD_TAG + " " + bench.json.dumps(rec) + "\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.stored_traffic("opt13b_decode", None) is None
    rec["sources_sha256"] = bench.kernel_sources_sha()
    (tmp_path / "old.md").write_text("`" + bench.RECORD_TAG + " " + bench.json.dumps(rec) + "`\n")
    assert bench.stored_traffic("opt13b_decode", None) == 1
