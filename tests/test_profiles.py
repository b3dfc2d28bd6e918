"""The rocprofv3 summaries under profiles/ belong to the library as built now.

Every kernel-duration summary, traffic record and counter table names the
hash of the kernel source and compiler flags it was taken on (bench.py's
source_sha); the bench reports a traffic record only while that hash is
unchanged. These checks fail as soon as the kernels change without the
profiles being taken again, and check that each summary carries the
command that produced it (a rocprofv3 run of bench.py).
"""
from __future__ import annotations

import glob
import json
import os
import re

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROF = os.path.join(ROOT, "profiles")


def test_every_summary_names_the_current_build():
    sha = bench.source_sha()
    mds = sorted(glob.glob(os.path.join(PROF, "*.md")))
    jsons = sorted(glob.glob(os.path.join(PROF, "*_traffic.json")))
    assert mds and jsons
    for f in mds:
        text = open(f, encoding="utf-8").read()
        hashes = set(re.findall(r"`([0-9a-f]{16})`", text))
        assert hashes == {sha}, (os.path.basename(f), hashes, sha)
        assert "rocprofv3 " in text and "python3 bench.py" in text, os.path.basename(f)
    for f in jsons:
        rec = json.load(open(f))
        assert rec["source_sha"] == sha, os.path.basename(f)
        assert all(c.startswith("rocprofv3 --pmc ") and "python3 bench.py" in c for c in rec["commands"])
        # FETCH counted what the call reads: at least the algorithmic bytes, within a few percent
        # above them (the merge kernel's partials), except the tiny launch-bound call
        ratio = rec["fetch_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"]
        assert 0.99 <= ratio <= (1.7 if rec["workload"] == "mqa-1k" else 1.1), (os.path.basename(f), ratio)


def test_traffic_record_name_matches_the_bench_tag():
    """bench.py looks a record up as decode_<workload>[-paged<P>][-t<T>][-fp8|-int8][-w<W>]
    _traffic.json; each record's workload and page size agree with its name."""
    for f in glob.glob(os.path.join(PROF, "*_traffic.json")):
        rec = json.load(open(f))
        tag = os.path.basename(f)[len("decode_"):-len("_traffic.json")]
        assert tag.startswith(rec["workload"]), (tag, rec["workload"])
        if rec["page_size"]:
            assert f"-paged{rec['page_size']}" in tag
        else:
            assert "-paged" not in tag


def test_design_notes_quote_the_current_build():
    text = open(os.path.join(ROOT, "DESIGN.md"), encoding="utf-8").read()
    quoted = set(re.findall(r"build hash `([0-9a-f]{16})`", text))
    assert quoted == {bench.source_sha()}, quoted
