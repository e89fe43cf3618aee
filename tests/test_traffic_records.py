"""The committed counter records: every record names kernels whose sources
are known, and those sources exist (a record holds while they are unchanged)."""

import json
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_every_record_names_known_kernels_and_existing_sources():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
        recs = json.load(fh)
    assert recs
    for key, rec in recs.items():
        for name in rec["kernels"].split(","):
            assert name in bench.KERNEL_SOURCES, (key, name)
        for rel in rec["sources_sha256"]:
            assert os.path.exists(os.path.join(ROOT, rel)), (key, rel)
        assert os.path.exists(os.path.join(ROOT, rec["summary"])), key


def test_every_kernel_source_list_exists():
    for name, files in bench.KERNEL_SOURCES.items():
        for f in files + bench._COMMON_SOURCES:
            assert os.path.exists(os.path.join(ROOT, bench.CSRC, f)), (name, f)
