"""Golden fixtures: the pages' printed numbers, and a regression file of oracle verdicts."""
import json
import os

import numpy as np
import pytest

import workloads
from oracle import svref

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_pages_mal_counts_the_extra_token():
    """With depth D, the printed acceptance rates and mean accepted lengths satisfy
    MAL = 1 + D * rate: MAL counts the correction/bonus token (n_out = tau + 1) and the
    acceptance rate is E[tau] / D -- the conventions the verifier's outputs follow."""
    rows = [l.split() for l in open(os.path.join(GOLD, "pages_mtp_numbers.txt")) if l.strip() and not l.startswith("#")]
    assert len(rows) == 2
    for _, rate, mal, d in rows:
        assert abs(1 + int(d) * float(rate) - float(mal)) < 0.005  # printed to 2 decimals


def test_oracle_n_out_convention():
    v = workloads.make_verify_inputs("tiny", device="cpu", T=1.0)
    res = svref.verify_batch(workloads.to_oracle(v.target), workloads.to_oracle(v.draft),
                             v.draft_tokens.numpy(), 1.0, "f32", seed=0)
    assert (res["n_out"] == res["accept_len"] + 1).all()


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_tiny_regression(T):
    gold = json.load(open(os.path.join(GOLD, "tiny_verify.json")))[f"T={T}"]
    v = workloads.make_verify_inputs("tiny", device="cpu", T=T)
    assert v.draft_tokens.numpy().tolist() == gold["draft_tokens"]
    res = svref.verify_batch(workloads.to_oracle(v.target), workloads.to_oracle(v.draft),
                             v.draft_tokens.numpy(), T, "f32", seed=v.seed, step=0)
    np.testing.assert_allclose(res["alpha"], gold["alpha"], rtol=1e-12)
    np.testing.assert_allclose(res["lse_t"], gold["lse_t"], rtol=1e-12)
    assert res["accept"].tolist() == gold["accept"]
    assert res["accept_len"].tolist() == gold["accept_len"]
    assert res["out_tokens"].tolist() == gold["out_tokens"]
    assert res["amax_t"].tolist() == gold["amax_t"]
