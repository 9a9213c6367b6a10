"""Host-side logic of the benchmark and of the counter summary (no GPU):
the one-GPU contract of bench.py, its error line without a GPU, the
copy-probe calibration of FETCH_SIZE / WRITE_SIZE, and the rule that stored
traffic figures go stale when the attention sources change."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def run(args, timeout=300):
    return subprocess.run([sys.executable, *args], cwd=ROOT, capture_output=True, text=True, timeout=timeout)


def test_bench_refuses_more_than_one_gpu():
    r = run(["bench.py", "--gpus", "2"])
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "exactly one GPU" in line["error"] and line["n_gpus"] == 2


def test_bench_without_a_gpu_prints_an_error_line():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible: the benchmark would run")
    r = run(["bench.py"])
    assert r.returncode == 1
    assert json.loads(r.stdout.strip().splitlines()[-1]) == {"error": "no GPU visible"}


def write_counters(path, counter, rows):
    """rows: (dispatch id, kernel name, value in KiB); each value is split over
    two counter dimensions, which the summary must add back up."""
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, name, v in rows:
            for part in (0.25 * v, 0.75 * v):
                w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": part})


def test_pmc_summary_calibrates_by_the_copy_probe(tmp_path):
    # a 1 MiB copy reads back as 512 KiB fetched (scale 2) and 1024 KiB written
    # (scale 1); two main-pass dispatches (both modes) and four combines
    copy = "copy_probe_kernel(unsigned int*, unsigned int const*, unsigned long)"
    main0, main1 = "void orthrus::attn_stream<128, 4, 0, false>(orthrus::AttnArgs)", \
        "void orthrus::attn_stream<128, 4, 1, false>(orthrus::AttnArgs)"
    comb = "void orthrus::attn_combine_bf16<128, 4, 8, false>(orthrus::AttnArgs)"
    fetch = [(1, copy, 512), (2, main0, 100), (3, comb, 10), (4, comb, 12), (5, main1, 140), (6, comb, 10),
             (7, comb, 8)]
    write = [(1, copy, 1024), (2, main0, 20), (3, comb, 1), (4, comb, 1), (5, main1, 20), (6, comb, 1),
             (7, comb, 1)]
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    write_counters(fp, "FETCH_SIZE", fetch)
    write_counters(wp, "WRITE_SIZE", write)
    r = run(["-m", "diffusion_drafted_verification_amd.pmc_summary", "--fetch", str(fp), "--write", str(wp),
             "--copy-mib", "1", "--batch", "1", "--ctx", "8"])
    assert r.returncode == 0, r.stderr
    # per call: the mean main pass (120 KiB fetched) plus two combines (20 KiB
    # on average), fetched bytes doubled; writes 20 + 2 KiB, not scaled
    read = (120 + 2 * 10) * 1024 * 2
    wrote = (20 + 2 * 1) * 1024
    last = r.stdout.strip().splitlines()[-1]
    assert f"read {read:,} B + write {wrote:,} B = {read + wrote:,} B" in last, last
    assert "scale 2.0000" in r.stdout and "scale 1.0000" in r.stdout


def test_stored_traffic_goes_stale_with_the_sources(tmp_path):
    import bench
    csrc = tmp_path / "diffusion_drafted_verification_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.ATTN_SOURCES:
        (csrc / f).write_text(f"// {f}\n")
    store = tmp_path / bench.TRAFFIC_FILE
    store.write_text(json.dumps({"attn_source_sha256": bench.attn_source_sha(str(tmp_path)),
                                 "workloads": {"b1_ctx8192": {"hbm_bytes_per_call": 48743022}}}))
    assert bench.measured_traffic(str(tmp_path), 1, 8192) == 48743022
    assert bench.measured_traffic(str(tmp_path), 16, 8192) is None      # another workload
    (csrc / bench.ATTN_SOURCES[0]).write_text("// changed\n")
    assert bench.measured_traffic(str(tmp_path), 1, 8192) is None       # the kernel changed since
