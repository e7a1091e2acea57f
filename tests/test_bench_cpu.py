"""CPU tests of bench.py's host logic: the kernel-code hash that keys the stored counter
readings, the launch configuration the benchmark times, and its one-GPU contract."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_only_strips_comments_and_keeps_literals():
    src = ('int a = 1; // trailing comment\n'
           '/* a block\n   comment */ const char* s = "x // not a comment /* nor this */";\n'
           "char q = '\"'; char e = '\\'';   int   b;\n")
    assert bench._code_only(src) == ('int a = 1; const char* s = "x // not a comment /* nor this */"; '
                                     "char q = '\"'; char e = '\\''; int b;")


def test_kernel_code_hash_ignores_comments_but_not_code():
    path = os.path.join(ROOT, "paged_kv_cache_mla_amd", "csrc", "decode_gqa.hip")
    with open(path, encoding="utf-8") as fh:
        text = fh.read()
    commented = "// an added comment line\n" + text.replace("\n", "  // note\n", 3)
    assert bench._code_only(commented) == bench._code_only(text)
    changed = text.replace("kRescaleSlack = 8.f", "kRescaleSlack = 9.f", 1)
    assert changed != text
    assert bench._code_only(changed) != bench._code_only(text)


def test_kernel_hash_covers_each_workload_sources():
    hashes = {w: bench.kernel_hash(w) for w in ("gqa_32k", "mla_16k", "split_128k")}
    assert hashes["gqa_32k"] == hashes["split_128k"]      # same kernel sources and flags
    assert hashes["gqa_32k"] != hashes["mla_16k"]
    assert all(len(h) == 16 for h in hashes.values())


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_csv(path, header, rows):
    with open(path, "w") as fh:
        fh.write(",".join(f'"{h}"' for h in header) + "\n")
        for r in rows:
            fh.write(",".join(f'"{v}"' for v in r) + "\n")


def test_profile_summary_picks_the_decode_kernel_not_the_probe(tmp_path):
    """The gather probe is timed next to the decode kernel and may run longer in total; the
    summary's stored values must still be the decode kernel's, with the HBM bytes scaled by
    the copy calibration (FETCH_SIZE reads half a copy's bytes, WRITE_SIZE all of them)."""
    dec = "kvattn::gqa_decode_mfma_kernel<128, 4, 2, true>(kvattn::DecodeArgs)"
    probe = "void kvattn::gqa_probe_kernel<128, 4, 2, true>(kvattn::DecodeArgs, unsigned int*)"
    copy = bench.COPY_KERNEL
    stats, fetch, write = tmp_path / "stats", tmp_path / "fetch", tmp_path / "write"
    for d in (stats, fetch, write):
        d.mkdir()
    _write_csv(stats / "run_kernel_stats.csv",
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"],
               [[probe, 22, 22 * 171000, 171000, 40, 168000, 180000, 1],
                [dec, 20, 20 * 163000, 163000, 38, 157000, 170000, 1],
                [copy, 12, 12 * 700000, 700000, 20, 600000, 800000, 1]])
    big = 2 << 30
    hdr = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    _write_csv(fetch / "run_counter_collection.csv", hdr,
               [[copy, 1 << 20, "FETCH_SIZE", big / 2 / 1024], [dec, 4096, "FETCH_SIZE", 524800.0],
                [probe, 4096, "FETCH_SIZE", 524300.0]])
    _write_csv(write / "run_counter_collection.csv", hdr,
               [[copy, 1 << 20, "WRITE_SIZE", big / 1024], [dec, 4096, "WRITE_SIZE", 1056.0],
                [probe, 4096, "WRITE_SIZE", 1.0]])
    out = tmp_path / "summary.md"
    bench.summarize_profile("gqa_32k", str(fetch), str(write), str(stats), str(out), ["cmd"])
    vals = bench.read_profile_values(str(out))
    assert vals["kernel"] == "kvattn::gqa_decode_mfma_kernel<128, 4, 2, true>"
    assert vals["avg_duration_us"] == "163.00"
    assert abs(float(vals["fetch_factor"]) - 2.0) < 1e-9 and abs(float(vals["write_factor"]) - 1.0) < 1e-9
    assert int(vals["hbm_bytes_per_launch"]) == round(524800.0 * 1024 * 2 + 1056.0 * 1024)
    assert vals["kernel_hash"] == bench.kernel_hash("gqa_32k")


def test_counter_summary_records_the_kernel_hash(tmp_path):
    """Counter summaries carry the code hash of the sources they were taken on, like the
    trace summaries, so a reading can be tied to (or voided by) the current kernel."""
    dec = "kvattn::mla_decode_kernel<false>(kvattn::DecodeArgs, unsigned int*)"
    d = tmp_path / "pmc"
    d.mkdir()
    _write_csv(d / "run_counter_collection.csv",
               ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"],
               [[dec, 256, "MfmaUtil", 7.5], [dec, 256, "MfmaUtil", 6.5]])
    out = tmp_path / "counters.md"
    bench.summarize_counters("mla_16k", [str(d)], str(out), ["cmd"])
    text = out.read_text()
    assert "| 2 | 7 |" in text            # two dispatches, their average
    assert bench.read_profile_values(str(out))["kernel_hash"] == bench.kernel_hash("mla_16k")


def test_sanitized_build_instruments_host_code_only():
    """The sanitizer builds put -Xarch_host before every -fsanitize= (device code is compiled
    as usual), write to their own directory, and name the runtime to preload."""
    from paged_kv_cache_mla_amd import build as B
    flags = B._sanitize_flags(("address", "undefined"))
    for i, f in enumerate(flags):
        if f.startswith("-fsanitize="):
            assert flags[i - 1] == "-Xarch_host"
    assert B.sanitized_path(("thread",)) != B.OUT
    cmd = B.sanitizer_test_command(("thread",))
    assert "libclang_rt.tsan" in cmd and "KVATTN_LIB=" in cmd and "halt_on_error=1" in cmd
    assert "libclang_rt.asan" in B.sanitizer_test_command(("address", "undefined"))
