"""The HBM traffic gate on the committed counter summaries (profiles/*_counters.txt with a
traffic_over_algorithmic line): counted bytes (FETCH_SIZE + WRITE_SIZE scaled by a copy of known
size) over the bytes the method must move, per kernel, must stay under the stated limits, and
each summary must have been taken from the kernel source as it is now (a summary of older code
is no evidence; refresh it with the commands written in its header)."""
import os
import re

import pytest

from bench import source_hash

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")

# Traffic over algorithmic bytes, per launch, at the 16-sequence decode shapes:
#  - the indexer scan streams every key once and writes only candidate lists: 1.10 leaves room
#    for the lists, the query and the bounds;
#  - CSA attention writes a 64-head partial per split (12 splits of 3 tiles per sequence) and
#    reads rows, ids and q: measured 3.36;
#  - HCA attention: 15 splits per sequence over 8,320 rows: measured 1.48.
LIMITS = {
    "index_cand_scan_csa1m_b16": 1.10,
    "csa_attend_csa1m_b16": 3.6,
    "hca_attend_hca1m_b16": 1.6,
}


def _read(name):
    rec, src = {}, None
    with open(os.path.join(PROFILES, f"{name}_counters.txt")) as f:
        for ln in f:
            m = re.search(r"source_sha256_16 is .*?(csrc/\S+\.hip)", ln)
            if m:
                src = m.group(1)
            if "=" in ln and not ln.lstrip().startswith("#"):
                k, v = ln.split("=", 1)
                rec[k.strip()] = v.strip()
    return rec, src


@pytest.mark.parametrize("name", sorted(LIMITS))
def test_counted_traffic_within_limit_and_current(name):
    rec, src = _read(name)
    assert src, f"{name}: the summary does not name its source file"
    path = os.path.join(ROOT, "long_context_attention_03_amd", src)
    assert rec["source_sha256_16"] == source_hash(path), \
        f"{name}: counters were taken from another version of {src}"
    fetch = float(rec["fetch_size_kib_per_dispatch"]) * 1024 * float(rec["fetch_factor"])
    write = float(rec["write_size_kib_per_dispatch"]) * 1024 * float(rec["write_factor"])
    total = float(rec["hbm_bytes_per_launch"])
    assert abs(fetch + write - total) <= 1e-6 * total + 2, f"{name}: bytes do not add up"
    ratio = total / float(rec["algorithmic_bytes_per_launch"])
    assert abs(ratio - float(rec["traffic_over_algorithmic"])) < 1e-3
    assert ratio <= LIMITS[name], f"{name}: {ratio:.3f} x the algorithmic bytes > {LIMITS[name]}"


def test_every_counter_summary_is_gated():
    have = {f[:-len("_counters.txt")] for f in os.listdir(PROFILES)
            if f.endswith("_counters.txt") and "traffic_over_algorithmic" in open(
                os.path.join(PROFILES, f)).read()}
    assert have == set(LIMITS), have ^ set(LIMITS)
