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


def test_default_group_parts():
    assert bench.default_group_parts("gqa_32k") == 16
    assert bench.default_group_parts("mla_16k") == 4
    assert [bench.default_group_parts("split_128k", r) for r in (0.25, 0.5, 0.75)] == [4, 8, 1]
    assert bench.default_group_parts("split_128k", 0.3) == bench.GROUP_PARTS["split_128k"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
