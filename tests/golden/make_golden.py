"""Write tests/golden/tiny_verify.json: the oracle's verdicts on the tiny workload.

Calls only the CPU oracle (oracle/) on inputs from the seeded generator; run from the
repository root: ``python tests/golden/make_golden.py``.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402
from oracle import svref  # noqa: E402


def main():
    out = {}
    for T in (1.0, 0.0):
        v = workloads.make_verify_inputs("tiny", device="cpu", T=T)
        res = svref.verify_batch(workloads.to_oracle(v.target), workloads.to_oracle(v.draft),
                                 v.draft_tokens.numpy(), T, "f32", seed=v.seed, step=0)
        out[f"T={T}"] = {
            "draft_tokens": v.draft_tokens.numpy().tolist(),
            "alpha": res["alpha"].tolist(),
            "lse_t": res["lse_t"].tolist(),
            "lse_d": res["lse_d"].tolist(),
            "accept": res["accept"].tolist(),
            "accept_len": res["accept_len"].tolist(),
            "out_tokens": res["out_tokens"].tolist(),
            "amax_t": res["amax_t"].tolist(),
        }
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_verify.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
