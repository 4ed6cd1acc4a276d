"""Bitwise layout invariance: the same rows give the same bytes (mismatch_count = 0,
max_abs_diff = 0) whether they arrive as one packed training batch, ragged rollout batches, row
chunks, any token-tile width, permuted, or with the vocabulary split into shards and merged.

The pages compare training and rollout logprobs with an exact equality check, never a tolerance
(nxbn.cn blog, §4.4), and report mismatch_count and max_abs_diff (RL-Kernel v0.1.0 summary,
"AMD Instinct MI300X validation").
"""

import numpy as np
import pytest

import datagen
from tests.helpers import assert_bitwise, dev_bits, dev_i32, host, say

pytestmark = pytest.mark.gpu


def _layouts(T, ragged):
    return [
        dict(),
        dict(batch_sizes=ragged),
        dict(vocab_shards=2),
        dict(vocab_shards=4),
        dict(batch_sizes=ragged, vocab_shards=2),
        dict(batch_sizes=ragged, vocab_shards=4),
        dict(row_chunk=7),
        dict(token_tile=32),
        dict(token_tile=64),
        dict(token_tile=128),
        dict(token_tile=256),
        dict(row_chunk=max(1, T // 3), token_tile=32, vocab_shards=2),
    ]


def _run_all(rlk, lp, h, W, y, layouts, keys):
    import torch

    hd, Wd, yd = dev_bits(h), dev_bits(W), dev_i32(y)
    outs = []
    for lay in layouts:
        say(f"layout {lay}")
        o = lp.forward(hd, Wd, yd, **lay)
        outs.append({k: o[k] for k in keys})
    torch.cuda.synchronize()
    return outs


def test_tiny_training_vs_rollout_layouts(rlk):
    w = datagen.WORKLOADS["tiny"]
    h, W = datagen.hidden_bits(w), datagen.weight_bits(w)
    y = datagen.uniform_targets(w.T, w.V, w.cfg)
    ragged = datagen.tiny_layout()
    lp = rlk.Logprob(w.H, w.V)
    outs = _run_all(rlk, lp, h, W, y, _layouts(w.T, ragged), ("logp", "lse"))
    for o in outs[1:]:
        for k in ("logp", "lse"):
            assert_bitwise(o[k], outs[0][k], k)


@pytest.mark.parametrize("tau,ent,S", [(1.0, True, 4), (0.7, True, 4), (1.0, False, 8),
                                       (1.0, True, 2)])
def test_medium_layouts(rlk, tau, ent, S):
    T, H, V = 700, 320 * 2, 8 * 1111
    h, W, y = datagen.small_case(T, H, V, 170)
    y[::11] = -1
    ragged = datagen.ragged_sizes_cover(T, 1, 256, 170)
    lp = rlk.Logprob(H, V, vocab_segments=S, temperature=tau, entropy=ent)
    keys = ("logp", "lse", "entropy") if ent else ("logp", "lse")
    lays = [l for l in _layouts(T, ragged) if l.get("vocab_shards", 1) <= S]
    outs = _run_all(rlk, lp, h, W, y, lays, keys)
    for o in outs[1:]:
        for k in keys:
            assert_bitwise(o[k], outs[0][k], k)


def test_run_to_run_and_row_permutation(rlk):
    import torch

    T, H, V = 500, 256, 6000
    h, W, y = datagen.small_case(T, H, V, 180)
    lp = rlk.Logprob(H, V, entropy=True)
    perm = np.random.default_rng(3).permutation(T)
    say("repeat and permutation")
    a = lp.forward(dev_bits(h), dev_bits(W), dev_i32(y))
    b = lp.forward(dev_bits(h), dev_bits(W), dev_i32(y))
    c = lp.forward(dev_bits(h[perm]), dev_bits(W), dev_i32(y[perm]))
    torch.cuda.synchronize()
    for k in ("logp", "lse", "entropy"):
        assert_bitwise(a[k], b[k], k)
        assert_bitwise(host(a[k])[perm], host(c[k]), k)
