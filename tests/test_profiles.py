"""The rocprofv3 summaries under profiles/ belong to the library as built now.

Every kernel-duration summary, traffic record and counter table names the
hash of the code of the kernel source and its C header (comments left out)
and of the compiler flags it was taken on (bench.py's source_sha); the bench
reports a traffic record only while that hash is unchanged. These checks fail as soon as the kernels change without the
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


def test_hash_ignores_comments_and_nothing_else():
    """The hash leaves out what builds to nothing: comments of either form,
    comment-only lines, trailing blanks. Any edit of the code, of a literal
    (also one that holds comment markers) or of the indentation changes it."""
    base = (
        '#include "x.h"  // header\n'
        "/* block\n   comment */\n"
        "__global__ void k(int *p) {\n"
        '    asm volatile("s_nop 0 // not a comment" ::: "memory");\n'
        "    p[0] = 3; /* inline */ p[1] = '/';\n"
        "}\n"
    )
    same = [
        base.replace("// header", "// another header"),
        base.replace("/* block\n   comment */", "// one line now"),
        base.replace("/* inline */", "/* a longer\n inline comment */"),
        base.replace("{\n", "{  // opens\n\n// a new comment line\n"),
        base.replace("}\n", "}   \n"),
    ]
    differ = [
        base.replace("p[0] = 3", "p[0] = 4"),
        base.replace("// not a comment", "// still not one"),
        base.replace("'/'", "'*'"),
        base.replace("    p[0]", "  p[0]"),
        base.replace('"x.h"', '"y.h"'),
    ]
    ref = bench.code_text(base)
    assert "// not a comment" in ref and "'/'" in ref
    assert "header" not in ref and "block" not in ref and "inline" not in ref
    for s in same:
        assert bench.code_text(s) == ref, s
    for s in differ:
        assert bench.code_text(s) != ref, s


def _summary(tag: str) -> dict:
    text = open(os.path.join(PROF, f"decode_{tag}_kernel_stats.md"), encoding="utf-8").read()
    m = re.search(r"kernel time median ([\d.]+) µs \(mean [\d.]+; main kernel ([\d.]+) \+ merge kernel ([\d.]+)\)",
                  text)
    b = re.search(r"Algorithmic bytes per call ([\d,]+): [\d.]+ GB/s over the kernel time \(([\d.]+) of 8 TB/s\)",
                  text)
    s = re.search(r"schedule ([a-z-]+)", text)
    assert m and b and s, tag
    return {"call": float(m.group(1)), "main": float(m.group(2)), "merge": float(m.group(3)),
            "bytes": int(b.group(1).replace(",", "")), "frac": float(b.group(2)), "schedule": s.group(1)}


def test_design_results_table_matches_the_summaries():
    """Every row of the design notes' results table quotes its profile summary
    as rounded there: kernel µs (main + merge), algorithmic MB, frac, the
    schedule and, where a traffic record exists, FETCH / algorithmic bytes;
    and every kernel-duration summary has its row."""
    text = open(os.path.join(ROOT, "DESIGN.md"), encoding="utf-8").read()
    row = re.compile(r"^\| [^|]+ \| ([a-z-]+) \| ([\d,.]+) \| ([\d.]+) \(([\d.]+) \+ ([\d.]+)\) \| ([\d.]+) \| "
                     r"([\d.]+|–) \| `([\w-]+)` \|$", re.M)
    rows = row.findall(text)
    assert len(rows) >= 40
    seen = set()
    for sched, mb, call, main, merge, frac, fetch, tag in rows:
        s = _summary(tag)
        seen.add(tag)
        assert sched == s["schedule"], tag
        assert abs(float(mb.replace(",", "")) - s["bytes"] / 1e6) <= 0.051, (tag, mb)
        for quoted, key in ((call, "call"), (main, "main"), (merge, "merge")):
            assert abs(float(quoted) - s[key]) <= 0.051, (tag, key, quoted, s[key])
        assert abs(float(frac) - s["frac"]) <= 0.00051 + 1e-9, (tag, frac, s["frac"])
        tf = os.path.join(PROF, f"decode_{tag}_traffic.json")
        if fetch == "–":
            assert not os.path.exists(tf), tag
        else:
            rec = json.load(open(tf))
            ratio = rec["fetch_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"]
            assert abs(float(fetch) - ratio) <= 0.00051, (tag, fetch, ratio)
    stats = {os.path.basename(f)[len("decode_"):-len("_kernel_stats.md")]
             for f in glob.glob(os.path.join(PROF, "decode_*_kernel_stats.md"))}
    assert stats == seen, stats ^ seen


def test_status_table_quotes_results_table_values():
    """The status table at the top of the design notes repeats figures of the
    results table: every three-decimal fraction and every µs figure in it is
    one of the results table's fracs or call times (as rounded there)."""
    text = open(os.path.join(ROOT, "DESIGN.md"), encoding="utf-8").read()
    status = text[text.index("**Status at a glance**"):text.index("Rocprofv3 summaries:")]
    row = re.compile(r"^\| [^|]+ \| [a-z-]+ \| [\d,.]+ \| ([\d.]+) \([\d.]+ \+ [\d.]+\) \| ([\d.]+) \| "
                     r"(?:[\d.]+|–) \| `[\w-]+` \|$", re.M)
    calls, fracs = set(), set()
    for call, frac in row.findall(text):
        calls.add(call)
        fracs.add(frac)
    quoted_fracs = re.findall(r"(?<![\d.])(0\.\d{3})(?![\d])", status)
    quoted_us = re.findall(r"(\d+\.\d) µs", status)
    assert quoted_fracs and quoted_us
    assert set(quoted_fracs) <= fracs, set(quoted_fracs) - fracs
    assert set(quoted_us) <= calls, set(quoted_us) - calls
