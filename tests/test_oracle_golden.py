"""The oracle still reproduces its committed regression fixture."""
import json
import os
import sys

GOLD = os.path.join(os.path.dirname(__file__), "golden")
sys.path.insert(0, GOLD)


def test_oracle_reproduces_tiny_step_fixture():
    import make_oracle_golden as M
    with open(os.path.join(GOLD, "oracle_tiny_step.json")) as f:
        ref = json.load(f)
    got = M.compute()
    assert abs(got["loss"] - ref["loss"]) <= 1e-12 * abs(ref["loss"])
    for k, v in ref["grad_l2"].items():
        assert abs(got["grad_l2"][k] - v) <= 1e-10 * max(abs(v), 1e-30), k
    for k, v in ref["param_l2_after"].items():
        assert abs(got["param_l2_after"][k] - v) <= 1e-12 * max(abs(v), 1e-30), k


def test_pages_padding_fact():
    with open(os.path.join(GOLD, "pages_facts.json")) as f:
        facts = json.load(f)
    assert facts["padded_vocab_size"]["value"] % facts["padding_multiple"]["value"] == 0
    assert facts["padded_vocab_size"]["value"] >= facts["gpt2_vocab_size"]["value"]
