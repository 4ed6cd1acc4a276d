"""Shared test plumbing: moving datagen bytes to the GPU and comparing results.

Nothing here computes any part of the method; comparisons are element-wise.
"""

from __future__ import annotations

import json
import os
import sys

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def say(msg: str) -> None:
    """Name the case on stdout before a GPU step (flushed, so a dying box still shows it)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev_bits(a: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def dev_i32(a: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def bitwise_report(a: np.ndarray, b: np.ndarray) -> dict:
    """mismatch_count over raw bytes and max_abs_diff of two fp32 arrays (NaN == NaN bytes)."""
    ua = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    ub = np.ascontiguousarray(b, dtype=np.float32).view(np.uint32)
    mism = int(np.count_nonzero(ua != ub))
    with np.errstate(invalid="ignore"):
        d = np.abs(a.astype(np.float64) - b.astype(np.float64))
    d = d[np.isfinite(d)]
    return {"mismatch_count": mism, "max_abs_diff": float(d.max()) if d.size else 0.0}


def assert_bitwise(a, b, what: str = "") -> None:
    r = bitwise_report(host(a) if not isinstance(a, np.ndarray) else a,
                       host(b) if not isinstance(b, np.ndarray) else b)
    assert r["mismatch_count"] == 0 and r["max_abs_diff"] == 0.0, (what, r)


def diff_stats(got: np.ndarray, want: np.ndarray, active: np.ndarray | None = None) -> dict:
    g = np.asarray(got, dtype=np.float64)
    w = np.asarray(want, dtype=np.float64)
    if active is not None:
        g, w = g[active], w[active]
    d = np.abs(g - w)
    return {"max": float(d.max()), "mean": float(d.mean()), "p50": float(np.percentile(d, 50)),
            "p90": float(np.percentile(d, 90)), "p99": float(np.percentile(d, 99)), "n": int(d.size)}


def golden_targets(name: str) -> tuple[np.ndarray, dict]:
    y = np.load(os.path.join(GOLDEN, f"targets_{name}.npy"), allow_pickle=False)
    with open(os.path.join(GOLDEN, f"targets_{name}.json")) as f:
        meta = json.load(f)
    return y, meta
