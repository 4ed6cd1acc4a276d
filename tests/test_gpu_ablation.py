"""The selected-logprob ablation matrix (vime issue #45, "[Docs] RL-Kernel ablation-matrix manual
for post-training users": its matrix-semantics section defines the four cells P/R, R/P, P/P and
R/R, with R/R never left out; its report-field list names mismatch_count, the
logprob_abs_diff_{mean,max,p50,p90,p99} of active tokens and the wall times).

Training layout: the rows in one pass. Rollout layout: the same rows as ragged decode batches
over 4 vocab shards. R is this library; P is a plain framework LM head (bench.p_head: vendor
GEMM to bf16 logits, fp32 log-softmax, a vocab-parallel merge across the shards). R/R must be
bit for bit equal; P/P shows that the same comparison fails for a head without a fixed numeric
contract, so a zero in R/R is evidence rather than a check that cannot fail.
"""

import numpy as np
import pytest

import bench
import datagen
from tests.helpers import dev_bits, dev_i32, golden_targets, say

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _print(cells):
    for name, c in cells.items():
        print(name, {k: (round(v, 9) if isinstance(v, float) else v) for k, v in c.items()
                     if k not in ("actual_training_implementation",
                                  "actual_rollout_implementation")}, flush=True)


def test_matrix_tiny(rlk):
    import torch

    w = datagen.WORKLOADS["tiny"]
    h, W = datagen.hidden_bits(w), datagen.weight_bits(w)
    y = datagen.uniform_targets(w.T, w.V, w.cfg)
    y[5::9] = -1
    sizes = datagen.tiny_layout()
    say("ablation matrix, tiny workload")
    lp = rlk.Logprob(w.H, w.V, vocab_segments=4)
    import oracle

    ref = oracle.logprob(h, W, y)["logp"]
    m = bench.ablation_matrix(rlk, np, torch, lp, dev_bits(h), dev_bits(W), dev_i32(y), sizes,
                              4, ref)
    cells = m["cells"]
    _print(cells)
    assert set(cells) == {"R/R", "P/R", "R/P", "P/P"}
    rr = cells["R/R"]
    assert rr["mismatch_count"] == 0 and rr["max_abs_diff"] == 0.0
    assert rr["training_vs_oracle_max"] <= TOL and rr["rollout_vs_oracle_max"] <= TOL
    for c in cells.values():
        assert c["active_token_count"] == int((y >= 0).sum())
        assert c["step_wall_time_ms"] > 0.0
    # a mixed cell compares two different numerics: it must see the difference
    assert cells["R/P"]["mismatch_count"] > 0 and cells["P/R"]["mismatch_count"] > 0


def test_matrix_qwen3_head(rlk):
    """Qwen3-8B head rows (T=4096, H=4096, V=151936) against the rollout's 30 decode batches x
    4 shards. R/R: no bit differs. P/P: the plain head changes bits between the two layouts."""
    import torch

    w = datagen.WORKLOADS["qwen3_8b_head"]
    h, W = datagen.hidden_bits(w), datagen.weight_bits(w)
    y, meta = golden_targets("qwen3_8b_head")
    assert meta["sha256_hidden"] == datagen.sha256(h)
    ref = bench.reference_logp(np, "qwen3_8b_head")
    sizes = datagen.decode_layout(w.T)
    say("ablation matrix, qwen3_8b_head, 30 decode batches x 4 shards")
    lp = rlk.Logprob(w.H, w.V, vocab_segments=4)
    m = bench.ablation_matrix(rlk, np, torch, lp, dev_bits(h), dev_bits(W), dev_i32(y), sizes,
                              4, ref, reps=1)
    cells = m["cells"]
    _print(cells)
    rr, pp = cells["R/R"], cells["P/P"]
    assert rr["mismatch_count"] == 0 and rr["max_abs_diff"] == 0.0
    assert rr["training_vs_oracle_max"] <= TOL and rr["rollout_vs_oracle_max"] <= TOL
    assert pp["mismatch_count"] > 0, "the plain head kept every bit across layouts"
    assert pp["training_vs_oracle_max"] <= 2e-3  # bf16 logits: ~1e-3 from the oracle
