"""Benchmark: batched draft verification on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--mode stoch|greedy]

A step is one sv_verify_batch call over the DFly block workload (B=64 requests, block of
16 drafts, V=131072, bfloat16 logits, T=0.9): temperature softmax of both rows, alpha,
accept test, first-reject scan and correction/bonus draw, all in the HIP kernels.  Inputs
are resident in HBM before timing starts and rotate through two copies (1.1 GB > 2x the
256 MB Infinity Cache) so every step reads from HBM.  --workload mtp | budget | e2e | e2e_bwd
| sample measure the other workloads (MTP chat verify, budget allocation + ragged verify, the
L_e2e objective and its gradient in the drafter logits, draft tokens and confidences) the
same way.

Prints one JSON line (rank 0).  `value` is verified draft positions per second.  The
`roofline` object divides the algorithmic bytes of one launch (2 * V * 2 bytes per
verified position, plus V * 2 for the bonus row of each fully accepted request) by the
launch's average duration: HIP events on the launch stream bracket the timed launches,
which run back to back, and the region's time is divided by their number.

Before the warm-up calls, the plain read-only streaming kernel (sv_stream_read) reads a
4 GiB buffer STREAM_PASSES times: its bandwidth is reported as the achievable reference
(`extra.stream_read`), and it leaves the device at its sustained clocks, so the timed calls
measure the kernels rather than the power-management ramp of an idle device.  The timed
region itself holds exactly --steps full calls.  Verification steps are issued through the
binding's prepared call (arguments marshalled once); `extra.host_issue_us_per_step` is the
host time of one issue.  The oracle leg (`cpu_baseline`) also compares one GPU call with the
oracle on every request of the batch (`extra.parity`).
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
    # the sources of the verification kernel (members and finalize workgroups) and its launch code
    for rel in ["draft_verification_softmax_amd/csrc/sv_device.hpp", "draft_verification_softmax_amd/csrc/team_device.hpp",
                "draft_verification_softmax_amd/csrc/team_kernel.hip", "draft_verification_softmax_amd/csrc/team.hpp"]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "verify_dfly_traffic.json")
COPY_BYTES = 1 << 30
STREAM_BYTES = 4 << 30
STREAM_PASSES = 12


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
    t = profiling.traffic(fetch, write, copy_fetch, copy_write, COPY_BYTES, ["stream_kernel"])
    per = {k: t[k] for k in ["stream_kernel"]}
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


def stream_reference(torch, sv, stream):
    """Achieved bandwidth of the read-only streaming kernel over STREAM_BYTES (first two passes
    untimed), timed with events on the launch stream."""
    buf = torch.empty(STREAM_BYTES, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for _ in range(2):
        sv.sv_stream_read(buf, sink, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(STREAM_PASSES):
        sv.sv_stream_read(buf, sink, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) / 1e3 / STREAM_PASSES
    del buf
    return {"GB/s": round(STREAM_BYTES / s / 1e9, 1), "bytes": STREAM_BYTES, "passes": STREAM_PASSES,
            "frac_of_peak": round(STREAM_BYTES / s / 1e9 / HBM_PEAK_GBS, 4)}


def host_info():
    """The host the oracle runs on: logical CPUs the process may use, and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_count": os.cpu_count(), "usable_cpus": usable, "model": model}


def parity_check(gpu_out, oracle_out, tn, dn, dtype, T, L=None):
    """Every request of one GPU call against the oracle's call on the same inputs, seed and
    step (the comparison the GPU tests make): counts of requests compared, near-threshold
    cases and mismatches outside the bands."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import parity

    g = {k: (None if v is None else v.cpu().numpy()) for k, v in gpu_out.items()}
    B = oracle_out["alpha"].shape[0]
    rep = {"requests": 0, "near_accept": 0, "near_token": 0, "mismatches": 0}
    for r in range(B):
        rep["requests"] += 1
        try:
            one = parity.compare_verify(g, oracle_out, tn, dn, dtype, T, check=[r], L=L, label="bench")
        except AssertionError as e:
            rep["mismatches"] += 1
            rep.setdefault("first_mismatch", f"request {r}: {str(e)[:200]}")
            continue
        rep["near_accept"] += one["near_accept"]
        rep["near_token"] += one["near_token"]
    return rep


def _oracle_time(fn):
    t0 = time.perf_counter()
    fn()
    return time.perf_counter() - t0


def cpu_baseline_verify(inputs, T, seed, draft_len=None, what="DFly", gpu_call=None):
    """The oracle, as it stands, on the whole batch (single thread); then, when gpu_call is
    given (a function of (seed, step) returning the GPU outputs of the same inputs), one GPU
    call at the oracle's seed and step compared with it request by request."""
    import workloads
    from oracle import svref

    tn, dn = workloads.to_oracle(inputs.target), workloads.to_oracle(inputs.draft)
    toks = inputs.draft_tokens.cpu().numpy()
    dl = None if draft_len is None else draft_len.cpu().numpy()
    B, K = toks.shape
    dtype = "bf16" if inputs.target.dtype.__str__().endswith("bfloat16") else "f32"
    res = {}
    dt = _oracle_time(lambda: res.update(o=svref.verify_batch(tn, dn, toks, T, dtype, seed=seed, draft_len=dl,
                                                              diagnostics=True)))
    npos = int(dl.sum()) if dl is not None else B * K
    out = {"value": npos / dt, "unit": "positions/s", "cores": 1, "kind": "oracle",
           "sample": f"whole {what} batch: {npos} verified positions of {B} requests, V={tn.shape[-1]}, T={T}, "
                     f"one pass, {dt:.1f} s single-threaded",
           "host": host_info()}
    par = None
    if gpu_call is not None:
        par = parity_check(gpu_call(seed, 0), res["o"], tn, dn, dtype, T, L=dl)
    return out, par


def cpu_baseline_e2e(target, draft, T, n_i=256):
    """The oracle's L_e2e on the first n_i positions (all D depths) of the set, single thread."""
    import workloads
    from oracle import svref

    tn, dn = workloads.to_oracle(target[:n_i]), workloads.to_oracle(draft[:n_i])
    D = target.shape[1]
    dt = _oracle_time(lambda: svref.tv_e2e_loss(tn, dn, T, "bf16"))
    return {"value": n_i * D / dt, "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n_i} of {target.shape[0]} positions x D={D}, V={target.shape[2]}, "
                      f"{dt:.1f} s single-threaded"}


def cpu_baseline_e2e_bwd(target, draft, T, n_i=64):
    """The oracle's L_e2e gradient on the first n_i sequences (all D depths), single thread."""
    import workloads
    from oracle import svref

    tn, dn = workloads.to_oracle(target[:n_i]), workloads.to_oracle(draft[:n_i])
    D = target.shape[1]
    dt = _oracle_time(lambda: svref.tv_e2e_backward(tn, dn, T, "bf16"))
    return {"value": n_i * D / dt, "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n_i} of {target.shape[0]} sequences x D={D}, V={target.shape[2]}, "
                      f"{dt:.1f} s single-threaded"}


def cpu_baseline_sample(draft, T, seed, n_rows=256):
    """The oracle's draft sampling on the first n_rows drafter rows, single thread."""
    import workloads
    from oracle import svref

    B, K, V = draft.shape
    nb = max(1, n_rows // K)
    dn = workloads.to_oracle(draft[:nb])
    dt = _oracle_time(lambda: svref.sample_drafts(dn, T, "bf16", seed=seed))
    return {"value": nb * K / dt, "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": f"first {nb} of {B} requests x {K} drafter rows, V={V}, {dt:.1f} s single-threaded"}


class Timed:
    """Times `step(i)` over n launches with HIP events on the launch stream.

    The n timed launches run back to back between two events, as a serving loop issues
    them: the average launch duration is the region's time over n.  The per-launch spread
    (p10 / median / p90) comes from a second pass of up to 200 launches with an event pair
    around each, which adds a few microseconds of event overhead to every launch it times."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def run(self, step, warmup, n):
        torch = self.torch
        self.warmup, self.n = warmup, n
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        t_all0, t_all1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t_all0.record(self.stream)
        for i in range(n):
            step(warmup + i)
        issue1 = time.perf_counter()
        t_all1.record(self.stream)
        torch.cuda.synchronize()
        self.wall = time.perf_counter() - wall0
        self.host_issue_us = (issue1 - wall0) / n * 1e6
        self.total_ms = t_all0.elapsed_time(t_all1)
        self.avg_launch_s = self.total_ms / n / 1e3
        m = min(n, 200)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(m)]
        for i in range(m):
            ev[i][0].record(self.stream)
            step(warmup + n + i)
            ev[i][1].record(self.stream)
        torch.cuda.synchronize()
        self.per_launch_ms = [a.elapsed_time(b) for a, b in ev]
        return self

    def percentiles_us(self):
        """p10 / median / p90 of the per-launch event times (second pass), in microseconds."""
        xs = sorted(self.per_launch_ms)
        pick = lambda f: round(xs[min(len(xs) - 1, int(f * (len(xs) - 1) + 0.5))] * 1e3, 2)
        return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9)}


def bench_verify(args, sv, workloads, torch, name):
    """dfly | mtp | budget: sv_verify_batch (after sv_alloc_verify_budget for budget)."""
    dev = "cuda"
    T = 0.9 if args.mode == "stoch" else 0.0
    conf = None
    N = None
    if name == "budget":
        base, conf, N = workloads.make_budget_inputs(device=dev, T=T)
    else:
        base = workloads.make_verify_inputs(name, device=dev, T=T)
    B, K1, V = base.target.shape
    K = K1 - 1
    ncopy = args.copies if args.copies else {"dfly": 2, "mtp": 24, "budget": 4}[name]
    copies = [base] + [workloads.VerifyInputs(base.target.clone(), base.draft.clone(), base.draft_tokens.clone(),
                                              base.T, base.seed, base.name) for _ in range(ncopy - 1)]
    ws = sv.Workspace(dev).get(B, K, V)
    stream = torch.cuda.current_stream()
    out = None
    alloc = None
    if conf is not None:
        # the allocation writes into fixed buffers, which the prepared selected-row calls read
        alloc = sv.sv_alloc_verify_budget(conf, N)
        n_rows = min(N, B * K)
    preps = []
    for c in copies:
        if conf is not None:
            p = sv.PreparedVerify(c.target, c.draft, c.draft_tokens, T, seed=c.seed, draft_len=alloc[0],
                                  row_list=alloc[2], n_rows=n_rows, workspace=ws, out=out, stream=stream)
        else:
            p = sv.PreparedVerify(c.target, c.draft, c.draft_tokens, T, seed=c.seed, workspace=ws, out=out,
                                  stream=stream)
        out = p.out
        preps.append(p)

    def step(i):
        if conf is not None:
            # allocation, then verification laid out over the selected rows only
            sv.sv_alloc_verify_budget(conf, N, out=alloc, stream=stream)
        preps[i % len(preps)].launch(i)

    ref = stream_reference(torch, sv, stream)
    tm = Timed(torch, stream).run(step, args.warmup, args.steps)
    # the draws differ per step (the step counter keys the generator): replay the timed steps
    # untimed to count the fully accepted requests of each
    n_full = []
    taus = []
    lens_h = alloc[0].cpu() if alloc is not None else torch.full((B,), K, dtype=torch.int32)
    for i in range(args.steps):
        step(args.warmup + i)
        tau = out["accept_len"].cpu()
        n_full.append(int((tau == lens_h).sum()))
        taus.append(float(tau.float().mean()))
    npos = int(lens_h.sum())
    alg_bytes = npos * 2 * V * 2 + (sum(n_full) / len(n_full)) * V * 2
    achieved = alg_bytes / tm.avg_launch_s / 1e9
    # warm cache: the same calls on one input copy (its rows partly still in the 256 MB
    # Infinity Cache from the call before), reported apart from the cache-cold figure
    warm = Timed(torch, stream).run(lambda i: preps[0].launch(i), args.warmup, args.steps)
    extra_t = {"warm_cache": {"avg_launch_us": round(warm.avg_launch_s * 1e6, 2),
                              "GB/s_algorithmic": round(alg_bytes / warm.avg_launch_s / 1e9, 1),
                              "note": "one input copy reused by every call; not the headline"},
               "stream_read": ref, "host_issue_us_per_step": round(tm.host_issue_us, 2)}
    cpu = None
    if not args.no_cpu_baseline:
        what = {"dfly": "DFly", "mtp": "MTP chat", "budget": "budget-selected ragged"}[name]

        def gpu_call(seed, step_):
            if conf is not None:
                sv.sv_alloc_verify_budget(conf, N, out=alloc, stream=stream)
            preps[0].launch(step_, seed=seed)
            torch.cuda.synchronize()
            return out

        cpu, par = cpu_baseline_verify(base, T, base.seed, draft_len=alloc[0] if alloc is not None else None,
                                       what=what, gpu_call=gpu_call)
        extra_t["parity"] = par
    if conf is not None:
        # the D-cut choice of the budget from a cost table (linear here: a fixed part plus a
        # per-position part, in microseconds), timed on its own
        cost = (40.0 + 0.05 * torch.arange(B * K + 1, device=dev, dtype=torch.float32)).contiguous()
        t2 = Timed(torch, stream).run(lambda i: sv.sv_dcut_verify_budget(conf, cost), 5, 50)
        n_c, _, _, _, _ = sv.sv_dcut_verify_budget(conf, cost)
        extra_t.update({"dcut_choice_us": round(t2.avg_launch_s * 1e6, 2), "dcut_chosen_n": int(n_c.item())})
    desc = {
        "dfly": f"DFly block verify: B={B} requests x block {K}, V={V}, bf16 logits",
        "mtp": f"MTP chat verify: B={B} requests x depth {K}, V={V}, bf16 logits",
        "budget": f"budget {N} of {B}x{K} by cumulative confidence, then verification of the selected rows: "
                  f"V={V}, bf16 logits (step = sv_alloc_verify_budget + sv_verify_selected)",
    }[name]
    mode = "T=0.9 stochastic" if T > 0 else "T=0 greedy"
    return dict(
        positions=npos, tm=tm, alg_bytes=alg_bytes, achieved=achieved, cpu=cpu,
        key=f"verify_rows_{args.mode}" if name == "dfly" else f"{name}_{args.mode}",
        config={"workload": f"{desc}, {mode}; cache-cold ({len(copies)} rotating input copies)",
                "B": B, "K": K, "V": V, "T": T, **({"budget_N": N} if N else {})},
        extra={"alpha_mean": round(float(out["alpha"].float().mean()), 4),
               "tau_mean": round(sum(taus) / len(taus), 3), "n_full_accept_mean": sum(n_full) / len(n_full),
               **extra_t})


def bench_e2e(args, sv, workloads, torch):
    dev = "cuda"
    target, draft, T = workloads.make_e2e_inputs(device=dev)
    I, D, V = target.shape
    ws = sv.Workspace(dev).get(I, D, V)
    alpha = torch.empty((I, D), dtype=torch.float32, device=dev)
    state = {}

    def step(i):
        state["loss"], _ = sv.sv_tv_e2e_loss(target, draft, T, alpha=alpha, workspace=ws)

    ref = stream_reference(torch, sv, torch.cuda.current_stream())
    tm = Timed(torch, torch.cuda.current_stream()).run(step, min(args.warmup, 3), min(args.steps, 10))
    npos = I * D
    alg_bytes = npos * 2 * V * 2
    cpu = None if args.no_cpu_baseline else cpu_baseline_e2e(target, draft, T)
    return dict(positions=npos, tm=tm, alg_bytes=alg_bytes, achieved=alg_bytes / tm.avg_launch_s / 1e9, cpu=cpu,
                key="e2e_alpha",
                config={"workload": f"end-to-end TV objective: |I|={I} positions x D={D}, V={V}, bf16 logits, "
                                    f"T={T} ({2 * target.numel() * 2 / 1e9:.1f} GB read per call)",
                        "I": I, "D": D, "V": V, "T": T},
                extra={"loss": float(state["loss"].item()), "alpha_mean": round(float(alpha.mean()), 4),
                       "stream_read": ref})


def bench_e2e_bwd(args, sv, workloads, torch):
    """sv_tv_e2e_backward on the L_e2e set (alpha from one untimed forward), bf16 gradient."""
    dev = "cuda"
    target, draft, T = workloads.make_e2e_inputs(device=dev)
    I, D, V = target.shape
    ws = sv.Workspace(dev).get(I, D, V)
    loss, alpha = sv.sv_tv_e2e_loss(target, draft, T, workspace=ws)
    grad = torch.empty((I, D, V), dtype=torch.bfloat16, device=dev)

    def step(i):
        sv.sv_tv_e2e_backward(target, draft, alpha, T, grad=grad, workspace=ws)

    ref = stream_reference(torch, sv, torch.cuda.current_stream())
    tm = Timed(torch, torch.cuda.current_stream()).run(step, min(args.warmup, 3), min(args.steps, 10))
    npos = I * D
    alg_bytes = npos * V * (2 + 2 + 2)   # read both logit rows, write the gradient row (bf16)
    cpu = None if args.no_cpu_baseline else cpu_baseline_e2e_bwd(target, draft, T)
    gs = grad[:64].float()
    return dict(positions=npos, tm=tm, alg_bytes=alg_bytes, achieved=alg_bytes / tm.avg_launch_s / 1e9, cpu=cpu,
                key="e2e_backward",
                config={"workload": f"L_e2e gradient in the drafter logits: |I|={I} x D={D}, V={V}, bf16 logits "
                                    f"and gradient, T={T} ({alg_bytes / 1e9:.1f} GB moved per call)",
                        "I": I, "D": D, "V": V, "T": T},
                extra={"loss": float(loss.item()), "grad_abs_mean_first64": float(gs.abs().mean()),
                       "grad_row_sum_max_first64": float(gs.sum(-1).abs().max()), "stream_read": ref})


def bench_sample(args, sv, workloads, torch):
    """sv_sample_drafts over the DFly drafter rows (B=64 x 16, V=131072, bf16)."""
    dev = "cuda"
    T = 0.9 if args.mode == "stoch" else 0.0
    base = workloads.make_verify_inputs("dfly", device=dev, T=T)
    B, K, V = base.draft.shape
    ncopy = args.copies if args.copies else 2
    copies = [base.draft] + [base.draft.clone() for _ in range(ncopy - 1)]
    ws = sv.Workspace(dev).get(B, K, V)
    state = {}

    def step(i):
        state["tok"], state["conf"] = sv.sv_sample_drafts(copies[i % len(copies)], T, seed=base.seed, step=i,
                                                          workspace=ws)

    ref = stream_reference(torch, sv, torch.cuda.current_stream())
    tm = Timed(torch, torch.cuda.current_stream()).run(step, args.warmup, args.steps)
    npos = B * K
    alg_bytes = npos * V * 2
    cpu = None if args.no_cpu_baseline else cpu_baseline_sample(base.draft, T, base.seed)
    mode = "T=0.9 stochastic" if T > 0 else "T=0 greedy"
    return dict(positions=npos, tm=tm, alg_bytes=alg_bytes, achieved=alg_bytes / tm.avg_launch_s / 1e9, cpu=cpu,
                key=f"sample_{args.mode}",
                config={"workload": f"draft tokens and confidences: B={B} requests x {K} drafter rows, V={V}, "
                                    f"bf16 logits, {mode}; cache-cold ({ncopy} rotating input copies)",
                        "B": B, "K": K, "V": V, "T": T},
                extra={"conf_mean": round(float(state["conf"].mean()), 4), "stream_read": ref})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--mode", choices=["stoch", "greedy"], default="stoch")
    ap.add_argument("--workload", choices=["dfly", "mtp", "budget", "e2e", "e2e_bwd", "sample"], default="dfly",
                    help="dfly (default: the headline line), mtp, budget (allocation + ragged verify), e2e "
                         "(L_e2e forward), e2e_bwd (its gradient) or sample (draft tokens and confidences)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copies", type=int, default=0, help="rotating input copies (0: per-workload default)")
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

    if args.workload == "e2e":
        r = bench_e2e(args, sv, workloads, torch)
    elif args.workload == "e2e_bwd":
        r = bench_e2e_bwd(args, sv, workloads, torch)
    elif args.workload == "sample":
        r = bench_sample(args, sv, workloads, torch)
    else:
        r = bench_verify(args, sv, workloads, torch, args.workload)
    tm = r["tm"]
    n = tm.n
    digest = _source_digest()
    line = {
        "metric": METRIC,
        "value": r["positions"] * n / (tm.total_ms / 1e3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": tm.warmup,
        "ms_per_step": tm.total_ms / n,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": r["config"],
        "roofline": {
            "bound": "hbm",
            "achieved": round(r["achieved"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(r["achieved"] / HBM_PEAK_GBS, 4),
            "traffic": _traffic(r["key"], digest),
            "kernel": r["key"],
            "alg_bytes_per_launch": round(r["alg_bytes"]),
            "avg_launch_us": round(tm.avg_launch_s * 1e6, 2),
        },
        "cpu_baseline": r["cpu"],
        "extra": {"hbm_gbs": round(r["achieved"], 1), **r["extra"], "wall_s_timed_region": round(tm.wall, 4),
                  "launch_us": tm.percentiles_us(), "source_digest": digest},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
