"""Write the float64 oracle's outputs for every row of the full-size workloads.

For qwen3_8b_head, long_grpo and norm_head this script evaluates the oracle (``oracle.logprob``,
float64, never the HIP library) on all T rows with the stored targets of tests/golden, and writes
``reference_<workload>.npy``: float64 [3, T] holding logp, lse and entropy (entropy zeros where
the workload has none; padded rows are all zero, as the oracle defines them). The json beside it
records the sha256 of the input bytes and of the targets the values belong to, so a test can tell
whether they still match the generated inputs.

    python tests/golden/make_reference.py [workload ...]
"""

from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import datagen  # noqa: E402
import oracle  # noqa: E402

NAMES = ["qwen3_8b_head", "long_grpo", "norm_head"]


def make(name: str, block: int = 2048) -> None:
    w = datagen.WORKLOADS[name]
    t0 = time.time()
    h = datagen.hidden_bits(w)
    Wb = datagen.weight_bits(w)
    gamma_b = datagen.gamma_bits(w) if w.rmsnorm else None
    y = np.load(os.path.join(HERE, f"targets_{name}.npy"), allow_pickle=False)
    with open(os.path.join(HERE, f"targets_{name}.json")) as f:
        tmeta = json.load(f)
    assert tmeta["sha256_hidden"] == datagen.sha256(h), "targets belong to other hidden bytes"
    assert tmeta["sha256_W"] == datagen.sha256(Wb), "targets belong to another W"
    W64 = oracle.bf16_bits_to_f64(Wb)
    out = np.zeros((3, w.T), dtype=np.float64)
    for r0 in range(0, w.T, block):
        rows = np.arange(r0, min(w.T, r0 + block))
        r = oracle.logprob(h, W64, y, tau=w.tau, gamma_bits=gamma_b, rms_eps=w.rms_eps,
                           want_entropy=w.rmsnorm, rows=rows)
        out[0, rows] = r["logp"]
        out[1, rows] = r["lse"]
        if w.rmsnorm:
            out[2, rows] = r["entropy"]
        print(f"{name}: rows {rows[-1] + 1}/{w.T} ({time.time() - t0:.0f}s)", flush=True)
    meta = {
        "workload": name,
        "T": w.T, "H": w.H, "V": w.V, "tau": w.tau,
        "rows": ["logp", "lse", "entropy"],
        "entropy": bool(w.rmsnorm),
        "sha256_hidden": datagen.sha256(h),
        "sha256_W": datagen.sha256(Wb),
        "sha256_gamma": None if gamma_b is None else datagen.sha256(gamma_b),
        "sha256_targets": datagen.sha256(y),
        "sha256_values": datagen.sha256(out),
        "recipe": "oracle.logprob (float64) on every row with the stored targets",
    }
    np.save(os.path.join(HERE, f"reference_{name}.npy"), out)
    with open(os.path.join(HERE, f"reference_{name}.json"), "w") as f:
        json.dump(meta, f, indent=1)
    print(f"{name}: done in {time.time() - t0:.0f}s", flush=True)


if __name__ == "__main__":
    for n in (sys.argv[1:] or NAMES):
        make(n)
