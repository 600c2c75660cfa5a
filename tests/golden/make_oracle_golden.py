"""Writes tests/golden/oracle_tiny_step.json from the CPU oracle alone.

Regression fixture: the tiny configuration (vocab 512, context 64, 2 layers,
4 heads, 64 channels, B=4, T=64) with seeded perturbed parameters and uniform
tokens, one forward + backward + AdamW step (lr 1e-3, betas 0.9/0.999,
eps 1e-8, wd 0) in float64.  Run:  python tests/golden/make_oracle_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from gpt_transformer_lm_amd import synthetic as S  # noqa: E402

CFG = O.OracleConfig(vocab_size=512, max_seq_len=64, num_layers=2, num_heads=4, channels=64)


def compute():
    p = S.random_params(512, 512, 64, 2, 64, seed=2024, perturbed=True)
    p = {k: v.astype(np.float64) for k, v in p.items()}
    tok, tgt = S.uniform_batch(4, 64, 512, seed=2025)
    loss, grads, newp, _ = O.gpt2_step(p, tok, tgt, CFG, None, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    return {
        "loss": float(loss),
        "grad_l2": {k: float(np.linalg.norm(v)) for k, v in grads.items()},
        "param_l2_after": {k: float(np.linalg.norm(v)) for k, v in newp.items()},
    }


if __name__ == "__main__":
    out = compute()
    out["_source"] = ("written by tests/golden/make_oracle_golden.py from oracle/ only; "
                      "a regression fixture of the oracle, not a page value")
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny_step.json"), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
