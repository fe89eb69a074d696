"""The CPU oracle's C code (oracle/svref.c) built with address and undefined-behaviour
sanitizers and run on the tiny verification workload (and a small bfloat16 one), whose
outputs must equal the regular build's, and on budget allocations checked against a brute
force ranking."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import workloads
from oracle import svref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MAIN = os.path.join(ROOT, "tests", "cpp", "svref_sanitize_main.c")
ORACLE = os.path.join(ROOT, "oracle")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("asan") / "svref_sanitize")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-fast-math", "-ffp-contract=off", "-Wall", "-I", ORACLE,
                    "-o", out, MAIN, os.path.join(ORACLE, "svref.c"), "-lm"], check=True)
    return out


def _run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    res = subprocess.run([exe, *args], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0, f"exit {res.returncode}\n{res.stdout}\n{res.stderr[-4000:]}"


CASES = [("tiny", 1.0, None), ("tiny", 0.0, None), ("dfly", 0.9, dict(B=3, K=4, V=3000, seed=23))]


@pytest.mark.parametrize("name,T,shape", CASES)
def test_oracle_under_sanitizers_matches_regular_build(exe, tmp_path, name, T, shape):
    v = workloads.make_verify_inputs(name, device="cpu", T=T, **(shape or {}))
    dt = "bf16" if name == "dfly" else "f32"
    tn, dn = workloads.to_oracle(v.target), workloads.to_oracle(v.draft)
    x = v.draft_tokens.numpy().astype(np.int32)
    B, K = x.shape
    V = tn.shape[-1]
    dl = np.full(B, K, np.int32)
    if B > 1:
        dl[1] = K // 2
    d = str(tmp_path)
    with open(os.path.join(d, "params.txt"), "w") as f:
        f.write(f"{B} {K} {V} {1 if dt == 'bf16' else 0} {T!r} {v.seed} 2\n")
    for fname, a in [("target.bin", tn), ("draft.bin", dn), ("tokens.bin", x), ("draft_len.bin", dl)]:
        np.ascontiguousarray(a).tofile(os.path.join(d, fname))
    _run(exe, "verify", d)
    want = svref.verify_batch(tn, dn, x, T, dt, seed=v.seed, step=2, draft_len=dl)

    def rd(fname, dtype, shape):
        return np.fromfile(os.path.join(d, fname), dtype=dtype).reshape(shape)

    for key, dtype, shp in [("alpha", np.float64, (B, K)), ("accept", np.uint8, (B, K)), ("lse_t", np.float64, (B, K)),
                            ("lse_d", np.float64, (B, K)), ("amax_t", np.int32, (B, K)), ("amax_d", np.int32, (B, K)),
                            ("accept_len", np.int32, (B,)), ("out_tokens", np.int32, (B, K + 1)),
                            ("n_out", np.int32, (B,))]:
        np.testing.assert_array_equal(rd(key + ".bin", dtype, shp), want[key], err_msg=key)
    resid = rd("resid.bin", np.int32, (B,))
    np.testing.assert_array_equal(resid, svref.residual_sample(tn, dn, want["accept_len"], T, dt, seed=v.seed, step=2,
                                                               draft_len=dl))
    # the residual sampler at the verified lengths gives the verified correction token
    np.testing.assert_array_equal(resid, want["out_tokens"][np.arange(B), want["accept_len"]])
    if T > 0:
        loss, loss_from_alpha = np.fromfile(os.path.join(d, "e2e.bin"), dtype=np.float64)
        assert abs(loss - loss_from_alpha) <= 1e-12


def test_budget_under_sanitizers_matches_brute_force(exe):
    _run(exe, "budget")
