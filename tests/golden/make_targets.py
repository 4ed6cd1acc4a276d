"""Write the stored targets of the full-size workloads, sampled from the oracle's softmax.

The qwen3_8b_head, long_grpo and norm_head workloads draw each row's target from softmax(z / tau)
of that row's logits (tau = 1, 1, 0.7). This script computes those logits with the float64 oracle
only (never the HIP library), draws by inverse CDF with datagen's per-row uniforms, marks the
long_grpo padding rows with -1, and stores int32 arrays next to the sha256 of the input bytes so
that a reader can tell whether the stored targets still belong to the generated inputs.

    python tests/golden/make_targets.py [workload ...]
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


def make(name: str, row_chunk: int = 512) -> None:
    w = datagen.WORKLOADS[name]
    t0 = time.time()
    h = datagen.hidden_bits(w)
    Wb = datagen.weight_bits(w)
    gamma_b = datagen.gamma_bits(w) if w.rmsnorm else None
    u = datagen.target_uniforms(w.T, w.cfg)
    pad = datagen.pad_mask(w)
    W64 = oracle.bf16_bits_to_f64(Wb)
    gamma = None if gamma_b is None else oracle.bf16_bits_to_f64(gamma_b)
    y = np.full(w.T, -1, dtype=np.int32)
    for r0 in range(0, w.T, row_chunk):
        r1 = min(w.T, r0 + row_chunk)
        act = np.nonzero(~pad[r0:r1])[0] + r0
        if act.size == 0:
            continue
        x = oracle.bf16_bits_to_f64(h[act])
        if gamma is not None:
            x = oracle.rmsnorm_bf16(x, gamma, w.rms_eps)
        zp = oracle.logits(x, W64) / w.tau
        y[act] = oracle.sample_targets(zp, u[act])
        if (r0 // row_chunk) % 16 == 0:
            print(f"{name}: rows {r1}/{w.T} ({time.time() - t0:.0f}s)", flush=True)
    meta = {
        "workload": name,
        "T": w.T, "H": w.H, "V": w.V, "tau": w.tau,
        "sha256_hidden": datagen.sha256(h),
        "sha256_W": datagen.sha256(Wb),
        "sha256_gamma": None if gamma_b is None else datagen.sha256(gamma_b),
        "sha256_targets": datagen.sha256(y),
        "padded_rows": int((y < 0).sum()),
        "recipe": "inverse-CDF draw from softmax(z/tau) of float64 oracle logits, "
                  "uniforms from datagen.target_uniforms",
    }
    np.save(os.path.join(HERE, f"targets_{name}.npy"), y)
    with open(os.path.join(HERE, f"targets_{name}.json"), "w") as f:
        json.dump(meta, f, indent=1)
    print(f"{name}: done in {time.time() - t0:.0f}s", flush=True)


if __name__ == "__main__":
    for n in (sys.argv[1:] or NAMES):
        make(n)
