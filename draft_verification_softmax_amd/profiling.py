"""HBM traffic per launch from rocprofv3 counter runs (host-side parsing, no GPU).

rocprofv3 ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` report, per dispatch, the kilobytes
the L2 fetched from / wrote to memory.  The counters are calibrated against a plain
elementwise kernel of known size (it reads and writes ``copy_bytes`` bytes each), and the
calibrated figures are averaged per kernel name.
"""
import csv
import glob
import os
from collections import defaultdict


def _counter_csv(path):
    """``path`` is a counter_collection.csv or a directory holding one (searched below)."""
    if os.path.isdir(path):
        hits = sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True))
        if not hits:
            raise FileNotFoundError(f"no counter_collection.csv under {path}")
        return hits[-1]
    return path


def per_kernel(path, counter):
    """{kernel name: [value per dispatch]} for one counter (values as reported, KiB)."""
    vals = defaultdict(dict)
    with open(_counter_csv(path), newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            disp = row.get("Dispatch_Id") or row.get("Correlation_Id")
            name = row["Kernel_Name"]
            # a counter may come as several rows per dispatch (one per instance): sum them
            vals[name][disp] = vals[name].get(disp, 0.0) + float(row["Counter_Value"])
    return {k: list(v.values()) for k, v in vals.items()}


def _mean_for(table, match):
    xs = [x for name, v in table.items() if match in name for x in v]
    if not xs:
        raise KeyError(f"no dispatch of a kernel matching {match!r}")
    return sum(xs) / len(xs), len(xs)


def traffic(fetch, write, copy_fetch, copy_write, copy_bytes, kernels, copy_match="neg"):
    """Calibrated HBM bytes per launch for each kernel substring in ``kernels``.

    Returns {"fetch_scale", "write_scale", kernel: {"fetch_bytes", "write_bytes", "dispatches"}}.
    The scale of each counter is copy_bytes divided by what it reads for the copy kernel.
    """
    cf, _ = _mean_for(per_kernel(copy_fetch, "FETCH_SIZE"), copy_match)
    cw, _ = _mean_for(per_kernel(copy_write, "WRITE_SIZE"), copy_match)
    fs, ws = copy_bytes / cf, copy_bytes / cw
    tf, tw = per_kernel(fetch, "FETCH_SIZE"), per_kernel(write, "WRITE_SIZE")
    out = {"fetch_scale": fs, "write_scale": ws}
    for k in kernels:
        f, n = _mean_for(tf, k)
        w, _ = _mean_for(tw, k)
        out[k] = {"fetch_bytes": f * fs, "write_bytes": w * ws, "dispatches": n}
    return out
