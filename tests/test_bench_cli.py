"""Benchmark command line on the CPU: the one-GPU contract and the source hash
that keys the committed profile counters."""
import os
import re
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_kernel_sources_cover_every_local_include():
    """A profile's counters stay valid only while every source its kernel is built from is unchanged."""
    for family, files in bench.KERNEL_SOURCES.items():
        main = os.path.join(bench.CSRC, files[0])
        includes = set(re.findall(r'#include "(pa_[a-z_]+\.h)"', open(main).read()))
        assert includes <= set(files[1:]), (family, includes - set(files[1:]))
        assert len(bench.kernel_source_hash(family)) == 16


def test_committed_profiles_name_a_known_workload_and_family():
    from workloads import CONFIG_ORDER, make_config
    names = [f[len("pmc_"):-len(".md")] for f in os.listdir(bench.PROFILES) if f.startswith("pmc_")]
    assert names
    for name in names:
        assert name in CONFIG_ORDER, name
        text = open(os.path.join(bench.PROFILES, f"pmc_{name}.md")).read()
        assert re.search(r"kernel_source_sha256: [0-9a-f]{16}", text), name
        assert bench.kernel_family(make_config(name, values=False)) in bench.KERNEL_SOURCES


def test_committed_profiles_match_the_kernel_sources():
    """Every committed summary was measured on the kernel sources in the tree: its recorded
    source hash is today's hash of the sources of the kernel its workload runs on."""
    from workloads import make_config
    pat = re.compile(r"^(trace|pmc|mfma)_(.+)\.md$")
    seen = 0
    for f in sorted(os.listdir(bench.PROFILES)):
        m = pat.match(f)
        if not m:
            continue
        family = bench.kernel_family(make_config(m.group(2), values=False))
        text = open(os.path.join(bench.PROFILES, f)).read()
        got = re.search(r"kernel_source_sha256: ([0-9a-f]{16})", text)
        assert got, f
        assert got.group(1) == bench.kernel_source_hash(family), (f, family)
        seen += 1
    assert seen >= 30


def test_every_workload_has_full_size_parity():
    """Each benchmark workload is also a full-size parity case."""
    from workloads import CONFIG_ORDER
    src = open(os.path.join(ROOT, "tests", "test_gpu_parity.py")).read()
    full = re.search(r"FULL = \[(.*?)\]", src, re.S).group(1)
    assert sorted(re.findall(r'"([a-z0-9_]+)"', full)) == sorted(CONFIG_ORDER)
