"""HBM traffic per kernel launch from rocprofv3 counter runs (profiling support, not the path).

Two `rocprofv3 --pmc` runs of `bench.py --copy-calibration`, one with FETCH_SIZE and one with
WRITE_SIZE, give KiB per dispatch for every kernel. The benchmark's plain 256 MiB device copy has
known traffic (256 MiB read, 256 MiB written), so each counter is scaled by what it reads for that
copy. The summary records a digest of the kernel sources: the benchmark reports the traffic only
while the sources are unchanged.

    python -m jagged_attention_recommendation_amd.counters FETCH_DIR WRITE_DIR > summary.txt

A second summary reads one run of shader-sequencer counters (`--sq DIR`): per kernel family the
mean per dispatch of each counter and the MFMA busy fraction. SQ_VALU_MFMA_BUSY_CYCLES sums the
cycles in which a SIMD's matrix unit was busy over all 1024 SIMDs; GRBM_GUI_ACTIVE, as rocprofv3
reports it on MI355X, sums the GPU-busy clock over the 8 XCDs (a 137 us launch reads about
2.4e6, eight times its ~3e5 cycles). The busy fraction is therefore
SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024): the share of the launch's cycles in
which the average SIMD's matrix unit worked.
"""
from __future__ import annotations

import collections
import csv
import glob
import hashlib
import json
import os
import sys

COPY_BYTES = 256 << 20
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
# kernel families: the D = 128 direct-load kernels and the D = 32 / 64 / MX kernels
KERNELS = {"fwd": ("fwd_dl_kernel", "fwd_pp_kernel", "fwd_kernel"), "dq": ("dq_dl_kernel", "dq_kernel"),
           "dkdv": ("dkdv_dl_kernel", "dkdv_kernel")}
SIMDS = 1024  # MI355X: 256 compute units x 4 SIMDs
XCDS = 8      # accelerator complex dies; GRBM_GUI_ACTIVE is summed over them


def family(kernel_name):
    for short, subs in KERNELS.items():
        if any(sub in kernel_name for sub in subs):
            return short
    return None


def csrc_digest() -> str:
    """sha256 over the kernel sources (names and contents, sorted by name)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".h", ".hip", ".cpp")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def per_dispatch(run_dir):
    """{dispatch id: (kernel name, grid size, summed counter value in KiB)}"""
    rows = []
    for f in glob.glob(os.path.join(run_dir, "*counter_collection.csv")):
        rows += list(csv.DictReader(open(f)))
    val = collections.defaultdict(float)
    meta = {}
    for r in rows:
        val[r["Dispatch_Id"]] += float(r["Counter_Value"])
        meta[r["Dispatch_Id"]] = (r["Kernel_Name"], int(r["Grid_Size"]))
    return {d: (meta[d][0], meta[d][1], v) for d, v in val.items()}


def summarize(fetch_dir, write_dir):
    fetch, write = per_dispatch(fetch_dir), per_dispatch(write_dir)

    def copy_kib(d):
        # the largest copyBuffer dispatches are the 256 MiB calibration copies
        vals = sorted((v for k, g, v in d.values() if "copyBuffer" in k), reverse=True)[:3]
        return sum(vals) / len(vals)

    f_scale = (COPY_BYTES / 1024) / copy_kib(fetch)
    w_scale = (COPY_BYTES / 1024) / copy_kib(write)
    out = {"copy_fetch_kib": round(copy_kib(fetch), 1), "copy_write_kib": round(copy_kib(write), 1),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4), "kernels": {}}
    for short in KERNELS:
        fv = [v for k, g, v in fetch.values() if family(k) == short]
        wv = [v for k, g, v in write.values() if family(k) == short]
        if not fv or not wv:
            continue
        fk, wk = sum(fv) / len(fv), sum(wv) / len(wv)
        out["kernels"][short] = {"dispatches": len(fv), "fetch_kib": round(fk, 1),
                                 "write_kib": round(wk, 1),
                                 "bytes": round(fk * 1024 * f_scale + wk * 1024 * w_scale)}
    out["csrc_sha256"] = csrc_digest()
    return out


def summarize_sq(run_dir):
    """{family: {counter: mean per dispatch, ..., "dispatches": n, "mfma_busy_pct": x}}.
    GRBM counters are per-instance copies of one clock (max taken), SQ counters are summed."""
    rows = []
    for f in glob.glob(os.path.join(run_dir, "*counter_collection.csv")):
        rows += list(csv.DictReader(open(f)))
    vals = collections.defaultdict(list)
    names = {}
    for r in rows:
        vals[(r["Dispatch_Id"], r["Counter_Name"])].append(float(r["Counter_Value"]))
        names[r["Dispatch_Id"]] = r["Kernel_Name"]
    per = collections.defaultdict(dict)
    for (d, c), v in vals.items():
        per[d][c] = max(v) if c.startswith("GRBM") else sum(v)
    out = {}
    for short in KERNELS:
        ds = [d for d in per if family(names[d]) == short]
        if not ds:
            continue
        counters = sorted({c for d in ds for c in per[d]})
        mean = {c: sum(per[d].get(c, 0.0) for d in ds) / len(ds) for c in counters}
        mean["dispatches"] = len(ds)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in mean and mean.get("GRBM_GUI_ACTIVE", 0) > 0:
            mean["mfma_busy_pct"] = round(100.0 * mean["SQ_VALU_MFMA_BUSY_CYCLES"]
                                          / (mean["GRBM_GUI_ACTIVE"] / XCDS * SIMDS), 2)
        out[short] = mean
    return out


def load_summary(path):
    """The json record of a summary file, or None."""
    try:
        with open(path) as f:
            for line in f:
                if line.startswith("json: "):
                    return json.loads(line[len("json: "):])
    except OSError:
        return None
    return None


def main(argv):
    if argv[1] == "--sq":
        s = summarize_sq(argv[2])
        for k, v in s.items():
            items = ", ".join(f"{c}={v[c]:.4g}" for c in sorted(v) if c not in ("dispatches",))
            print(f"{k:5} dispatches={v['dispatches']}: {items}")
        print("json: " + json.dumps(s))
        return
    fetch_dir, write_dir = argv[1], argv[2]
    s = summarize(fetch_dir, write_dir)
    print(f"# calibration: the 256 MiB copy reads as {s['copy_fetch_kib']} KiB FETCH_SIZE "
          f"(scale {s['fetch_scale']}) and {s['copy_write_kib']} KiB WRITE_SIZE (scale {s['write_scale']})")
    print(f"{'kernel':8} {'dispatches':>10} {'FETCH_KiB':>12} {'WRITE_KiB':>12} {'scaled_MB':>10}")
    for k, v in s["kernels"].items():
        print(f"{k:8} {v['dispatches']:>10} {v['fetch_kib']:>12} {v['write_kib']:>12} {v['bytes'] / 1e6:>10.1f}")
    print("json: " + json.dumps(s))


if __name__ == "__main__":
    main(sys.argv)
