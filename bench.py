"""Benchmark: batched draft verification on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--mode stoch|greedy]

A step is one sv_verify_batch call over the DFly block workload (B=64 requests, block of
16 drafts, V=131072, bfloat16 logits, T=0.9): temperature softmax of both rows, alpha,
accept test, first-reject scan and correction/bonus draw, all in the HIP kernels.  Inputs
are resident in HBM before timing starts and rotate through two copies (1.1 GB > 2x the
256 MB Infinity Cache) so every step reads from HBM.

Prints one JSON line (rank 0).  `value` is verified draft positions per second.  The
`roofline` object divides the algorithmic bytes of one launch (2 * V * 2 bytes per
verified position, plus V * 2 for the bonus row of each fully accepted request) by the
launch's average duration, measured with HIP events on the launch stream.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "verified draft positions/s + HBM GB/s (% peak), B=64 block16 V=131072 bf16"


def _source_digest():
    h = hashlib.sha256()
    for rel in ["draft_verification_softmax_amd/csrc/specverify.hip", "draft_verification_softmax_amd/csrc/sv_device.hpp",
                "draft_verification_softmax_amd/csrc/team_kernel.hip", "draft_verification_softmax_amd/csrc/team.hpp"]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "verify_dfly_traffic.json")
COPY_BYTES = 1 << 30


def _traffic(kernel_key, digest):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they were taken
    on the current kernel source; else None."""
    try:
        d = json.load(open(TRAFFIC_JSON))
    except Exception:
        return None
    e = d.get(kernel_key)
    if not e or e.get("source_digest") != digest:
        return None
    return e.get("hbm_bytes_per_launch")


def copy_calibration(steps=5):
    """A plain elementwise kernel of known size (float32 negation: reads and writes
    COPY_BYTES each), timed with events; used to calibrate the HBM byte counters."""
    import torch
    x = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.neg(x, out=y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        torch.neg(x, out=y)
    e1.record()
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) / 1e3 / steps
    print(json.dumps({"copy_calibration": {"bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                                           "us": round(s * 1e6, 1), "GB/s": round(2 * COPY_BYTES / s / 1e9, 1)}}),
          flush=True)


def write_traffic(mode, fetch, write, copy_fetch, copy_write):
    """Fold two counter runs of bench.py (FETCH_SIZE, WRITE_SIZE) and two of
    --copy-calibration into profiles/verify_dfly_traffic.json (no GPU needed)."""
    from draft_verification_softmax_amd import profiling
    t = profiling.traffic(fetch, write, copy_fetch, copy_write, COPY_BYTES, ["stream_kernel", "finalize_kernel"])
    per = {k: t[k] for k in ["stream_kernel", "finalize_kernel"]}
    total = sum(v["fetch_bytes"] + v["write_bytes"] for v in per.values())
    try:
        d = json.load(open(TRAFFIC_JSON))
    except Exception:
        d = {}
    d[f"verify_rows_{mode}"] = {"source_digest": _source_digest(), "hbm_bytes_per_launch": round(total),
                                "fetch_scale": round(t["fetch_scale"], 5), "write_scale": round(t["write_scale"], 5),
                                "kernels": {k: {kk: round(vv) for kk, vv in v.items()} for k, v in per.items()}}
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(d, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(d[f"verify_rows_{mode}"]))


def cpu_baseline(inputs, T, seed):
    """The oracle, as it stands, on the whole batch (single thread)."""
    import numpy as np  # noqa: F401

    import workloads
    from oracle import svref

    tn, dn = workloads.to_oracle(inputs.target), workloads.to_oracle(inputs.draft)
    toks = inputs.draft_tokens.cpu().numpy()
    B, K = toks.shape
    t0 = time.perf_counter()
    svref.verify_batch(tn, dn, toks, T, "bf16", seed=seed)
    dt = time.perf_counter() - t0
    return {"value": B * K / dt, "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": f"whole DFly batch: {B} requests x {K} positions, V={tn.shape[-1]}, T={T}, "
                      f"one pass, {dt:.1f} s single-threaded"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--mode", choices=["stoch", "greedy"], default="stoch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copies", type=int, default=2)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only the known-size elementwise kernel used to calibrate byte counters")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="fold rocprofv3 counter outputs into the committed traffic summary and exit")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(args.mode, *args.write_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the verification path is data-parallel by request and needs no collective "
              "on one GPU's share; see the sharding note in the design document)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration()
        return

    import draft_verification_softmax_amd as sv
    import workloads

    dev = "cuda"
    T = 0.9 if args.mode == "stoch" else 0.0
    base = workloads.make_verify_inputs("dfly", device=dev, T=T)
    B, K1, V = base.target.shape
    K = K1 - 1
    copies = [base] + [workloads.VerifyInputs(base.target.clone(), base.draft.clone(), base.draft_tokens.clone(),
                                              base.T, base.seed, base.name) for _ in range(args.copies - 1)]
    ws = sv.Workspace(dev).get(B, K, V)
    out = None
    stream = torch.cuda.current_stream()

    def step(i):
        nonlocal out
        c = copies[i % len(copies)]
        out = sv.sv_verify_batch(c.target, c.draft, c.draft_tokens, T, seed=c.seed, step=i, workspace=ws,
                                 out=out, want_lse=True)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    n = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    t_all0, t_all1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_all0.record(stream)
    for i in range(n):
        ev[i][0].record(stream)
        step(args.warmup + i)
        ev[i][1].record(stream)
    t_all1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per_launch_ms = [a.elapsed_time(b) for a, b in ev]
    total_ms = t_all0.elapsed_time(t_all1)
    avg_launch_s = sum(per_launch_ms) / n / 1e3

    tau = out["accept_len"].cpu()
    n_full = int((tau == K).sum())
    alpha_mean = float(out["alpha"].float().mean())
    positions = B * K
    alg_bytes = positions * 2 * V * 2 + n_full * V * 2
    achieved = alg_bytes / avg_launch_s / 1e9
    digest = _source_digest()
    key = f"verify_rows_{args.mode}"
    traffic = _traffic(key, digest)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(base, T, base.seed)

    line = {
        "metric": METRIC,
        "value": positions * n / (total_ms / 1e3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": args.warmup,
        "ms_per_step": total_ms / n,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"DFly block verify: B={B} requests x block {K}, V={V}, bf16 logits, "
                        f"{'T=0.9 stochastic' if T > 0 else 'T=0 greedy'}; cache-cold ({len(copies)} rotating "
                        f"input copies)",
            "B": B, "K": K, "V": V, "T": T,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": key,
            "alg_bytes_per_launch": alg_bytes,
            "avg_launch_us": round(avg_launch_s * 1e6, 2),
        },
        "cpu_baseline": cpu,
        "extra": {
            "hbm_gbs": round(achieved, 1),
            "alpha_mean": round(alpha_mean, 4),
            "tau_mean": round(float(tau.float().mean()), 3),
            "n_full_accept": n_full,
            "wall_s_timed_region": round(wall, 4),
            "source_digest": digest,
        },
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
