"""Summarise rocprofv3 FETCH_SIZE / WRITE_SIZE counter runs of bench.py.

Usage (after two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of
`bench.py --no-graph --copy-probe-mib N ...` with `--output-format csv`):

    python -m diffusion_drafted_verification_amd.pmc_summary \
        --fetch <dir>/run_counter_collection.csv --write <dir>/run_counter_collection.csv \
        --copy-mib N --batch 1 --ctx 8192 [--update-json]

Both counters read in KiB per dispatch.  The plain device copy of N MiB
(`copy_probe_kernel`, which reads N MiB and writes N MiB exactly once) gives
the scale from counter units to bytes, so that

    HBM bytes per call = sum over the call's kernels of
        avg FETCH_SIZE * 1024 * (N MiB / copy FETCH bytes)
      + avg WRITE_SIZE * 1024 * (N MiB / copy WRITE bytes)

A block-attention call is one main-pass dispatch (`attn_stream` or
`attn_main`, either mask mode) plus, when the context is split, one
`attn_combine` dispatch; the per-call figure is the main-pass average plus
the combine average weighted by combine dispatches per main dispatch.  With `--update-json` the result is stored in
traffic_counters.json next to this file, keyed by the workload and stamped
with the hash of the attention kernel sources, so that a later change to the
kernel makes the stored figure stale.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
ATTN_SOURCES = ("block_attn.hip", "orthrus_device.h", "orthrus_host.h")


def attn_source_sha() -> str:
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(HERE, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_counter(path: str, counter: str) -> dict[str, list[float]]:
    """Kernel name -> per-dispatch values of `counter` (summed over the
    counter's dimensions within a dispatch)."""
    per_dispatch: dict[tuple[str, str], float] = defaultdict(float)
    with open(path, newline="") as fh:
        for row in csv.DictReader(fh):
            if row.get("Counter_Name") != counter:
                continue
            key = (row["Dispatch_Id"], row["Kernel_Name"])
            per_dispatch[key] += float(row["Counter_Value"])
    out: dict[str, list[float]] = defaultdict(list)
    for (_, name), v in sorted(per_dispatch.items(), key=lambda kv: int(kv[0][0])):
        out[name].append(v)
    return out


def short(name: str) -> str:
    name = name.split("(")[0]
    return name.replace("void ", "").strip()


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--fetch", required=True)
    p.add_argument("--write", required=True)
    p.add_argument("--copy-mib", type=int, required=True)
    p.add_argument("--batch", type=int, required=True)
    p.add_argument("--ctx", type=int, required=True)
    p.add_argument("--kv-bytes-per-call", type=int, default=0,
                   help="algorithmic KV bytes per call (default: ctx * batch * 4096)")
    p.add_argument("--update-json", action="store_true")
    a = p.parse_args()

    fetch = read_counter(a.fetch, "FETCH_SIZE")
    write = read_counter(a.write, "WRITE_SIZE")
    copy_bytes = a.copy_mib << 20

    def find(d, pat):
        return [k for k in d if pat in k]

    cf, cw = find(fetch, "copy_probe_kernel"), find(write, "copy_probe_kernel")
    if not cf or not cw:
        raise SystemExit("no copy_probe_kernel dispatch in the counter files")
    f_copy = sum(fetch[cf[0]]) / len(fetch[cf[0]]) * 1024
    w_copy = sum(write[cw[0]]) / len(write[cw[0]]) * 1024
    sf, sw = copy_bytes / f_copy, copy_bytes / w_copy

    # a call is one main-pass dispatch (either mask mode) plus, when the
    # context is split, one combine dispatch
    rows = []
    groups = {"main": [0, 0.0, 0.0], "combine": [0, 0.0, 0.0]}
    for name in sorted(set(fetch) | set(write)):
        if "attn_" not in name:
            continue
        fv, wv = fetch.get(name, []), write.get(name, [])
        fa = sum(fv) / len(fv) * 1024 * sf if fv else 0.0
        wa = sum(wv) / len(wv) * 1024 * sw if wv else 0.0
        rows.append((short(name), len(fv), fa, wa))
        gr = groups["combine" if "combine" in name else "main"]
        gr[0] += len(fv)
        gr[1] += fa * len(fv)
        gr[2] += wa * len(fv)
    n_main = groups["main"][0]
    if n_main == 0:
        raise SystemExit("no attention main-pass dispatch in the counter files")
    call_f = (groups["main"][1] + groups["combine"][1]) / n_main
    call_w = (groups["main"][2] + groups["combine"][2]) / n_main

    kv = a.kv_bytes_per_call or a.ctx * a.batch * 4096
    print(f"copy probe: {a.copy_mib} MiB; FETCH_SIZE reads {f_copy / 1024:.0f} KiB (scale {sf:.4f}), "
          f"WRITE_SIZE reads {w_copy / 1024:.0f} KiB (scale {sw:.4f})")
    print()
    print("| kernel | dispatches | HBM read B/dispatch | HBM write B/dispatch |")
    print("|---|---|---|---|")
    for n, c, fa, wa in rows:
        print(f"| `{n}` | {c} | {fa:,.0f} | {wa:,.0f} |")
    print()
    print(f"block-attention call (B{a.batch}, ctx {a.ctx}): read {call_f:,.0f} B + write {call_w:,.0f} B "
          f"= {call_f + call_w:,.0f} B; algorithmic KV bytes {kv:,} "
          f"(traffic / algorithmic = {(call_f + call_w) / kv:.3f})")

    if a.update_json:
        path = os.path.join(HERE, "traffic_counters.json")
        d = {}
        if os.path.exists(path):
            with open(path) as fh:
                d = json.load(fh)
        sha = attn_source_sha()
        if d.get("attn_source_sha256") != sha:
            d = {"attn_source_sha256": sha, "workloads": {}}
        d["workloads"][f"b{a.batch}_ctx{a.ctx}"] = {
            "hbm_bytes_per_call": int(round(call_f + call_w)), "read_bytes_per_call": int(round(call_f)),
            "write_bytes_per_call": int(round(call_w)), "copy_scale_fetch": round(sf, 5),
            "copy_scale_write": round(sw, 5), "algorithmic_kv_bytes": kv}
        with open(path, "w") as fh:
            json.dump(d, fh, indent=1, sort_keys=True)
            fh.write("\n")


if __name__ == "__main__":
    main()
