"""Consistency of the committed measurement records (CPU only): every counter
record in profiles/traffic.json names a kernel whose sources bench.py knows,
its summary file under profiles/ names the same kernel and the same source
hash, and its traffic figures add up."""
import json
import os
import re

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RECORDS = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
WORKLOADS = sorted(k for k, v in RECORDS.items() if isinstance(v, dict) and "kernel" in v)


def test_every_kernel_family_has_sources():
    for w in WORKLOADS:
        fam = RECORDS[w]["kernel"].split("<")[0]
        assert fam in bench.KERNEL_SOURCES, (w, fam)
        for p in bench.KERNEL_SOURCES[fam]:
            assert os.path.exists(os.path.join(ROOT, p)), p


@pytest.mark.parametrize("workload", WORKLOADS)
def test_summary_matches_record(workload):
    e = RECORDS[workload]
    kern = e["kernel"]
    path = os.path.join(ROOT, "profiles", f"{kern.split('<')[0]}_{workload}.md")
    text = open(path).read()
    assert text.startswith(f"# {kern} -- "), path
    m = re.search(r"Kernel sources hash \(bench\.py `source_hash`[^)]*\): `([0-9a-f]+)`", text)
    assert m and m.group(1) == e["source_hash"], path
    assert e["bytes_per_launch"] == pytest.approx(e["fetch_bytes"] + e["write_bytes"])
    # traffic is at least the algorithmic bytes (minus counter granularity)
    assert e["bytes_per_launch"] >= 0.98 * e["algorithmic_bytes"], workload
    # the summary's algorithmic bytes are the record's
    a = re.search(r"Algorithmic bytes per launch: ([\d,]+)", text)
    assert a and int(a.group(1).replace(",", "")) == e["algorithmic_bytes"], path
