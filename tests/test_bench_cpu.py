"""CPU checks of bench.py's contract and of the counter records it reports from
profiles/: a multi-GPU request is refused with a message, and every record was
taken on the kernel source that is in the tree now (the digest bench.py uses to
decide whether to report it), with figures that follow from its own trace."""
import glob
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

PEAK = 2.5e15


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


RECORDS = sorted(glob.glob(os.path.join(ROOT, "profiles", "counters_*.json")))


@pytest.mark.parametrize("path", RECORDS, ids=[os.path.basename(p) for p in RECORDS])
def test_counter_record_matches_current_source(path):
    with open(path) as f:
        rec = json.load(f)
    src = os.path.basename(rec["source_file"])
    assert rec["source_digest"] == bench.src_digest(src), \
        "%s was taken on another version of %s" % (os.path.basename(path), src)


@pytest.mark.parametrize("path", RECORDS, ids=[os.path.basename(p) for p in RECORDS])
def test_counter_record_fraction_follows_from_its_trace(path):
    with open(path) as f:
        rec = json.load(f)
    if "frac_of_bf16_peak_from_trace" not in rec:
        pytest.skip("bandwidth-bound kernel")
    useful = rec.get("useful_flop_per_launch", rec.get("useful_flop_per_step"))
    tr = rec["trace"]
    ms = tr.get("mean_ms", tr.get("sum_mean_ms"))
    assert rec["frac_of_bf16_peak_from_trace"] == pytest.approx(useful / (ms * 1e-3) / PEAK,
                                                                rel=1e-3)
    # the bench line printed by the traced run times the same step
    assert abs(rec["same_run_bench_line"]["rel_diff_step_time"]) < 0.05


def test_traffic_records_match_current_sources():
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
        rec = json.load(f)
    src = {"swa_fwd_prefill": "swa_tile_bf16.hip", "swa_fwd_varlen_gqa": "swa_tile_bf16.hip",
           "swa_prefill_chunk": "swa_tile_bf16.hip", "swa_decode": "swa_decode_bf16.hip"}
    for key, name in src.items():
        assert rec[key]["source_digest"] == bench.src_digest(name), key
        assert rec[key]["bytes_per_launch"] > 0
