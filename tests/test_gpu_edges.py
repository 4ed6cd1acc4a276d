"""Degenerate inputs on the GPU: no rows at all, empty decode batches between full ones, every
row padded, a single row, and a launch whose rows end one short of a row tile.

A rollout engine hands the recompute step whatever the scheduler produced, empty steps included
(nxbn.cn blog, §3.3: the rollout side recomputes logprobs from hidden states and tokens); the
answer for each row must not depend on how the rows were grouped (RL-Kernel v0.1.0 summary,
"Numeric execution contract").
"""

import numpy as np
import pytest

import datagen
import oracle
from tests.helpers import assert_bitwise, dev_bits, dev_i32, host, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("ent,rms", [(False, False), (True, True)])
def test_no_rows_is_a_no_op(rlk, ent, rms):
    import torch

    H, V = 256, 1000
    say(f"forward and backward with T = 0 (entropy={ent}, rmsnorm={rms})")
    lp = rlk.Logprob(H, V, entropy=ent, rmsnorm=rms)
    W = dev_bits(datagen.normal_bf16(V, H, 131, datagen.TID_W, scale=0.02))
    h = torch.empty((0, H), dtype=torch.int16, device="cuda")
    y = torch.empty((0,), dtype=torch.int32, device="cuda")
    g = dev_bits(datagen.normal_bf16(1, H, 131, datagen.TID_GAMMA, scale=0.1, mean=1.0)[0]) if rms else None
    o = lp.forward(h, W, y, gamma=g)
    torch.cuda.synchronize()
    assert o["logp"].numel() == 0 and o["lse"].numel() == 0
    assert lp.device_status(o["_workspace"]) == 0
    # no rows contribute to the gradients: grad_W (and grad_gamma) come back exactly zero
    z = torch.empty((0,), dtype=torch.float32, device="cuda")
    gr = lp.backward(h, W, y, z, z, entropy=o.get("entropy"), gamma=g)
    torch.cuda.synchronize()
    assert gr["grad_hidden"].shape == (0, H)
    assert int(torch.count_nonzero(gr["grad_W"])) == 0
    if rms:
        assert int(torch.count_nonzero(gr["grad_gamma"])) == 0


def test_empty_decode_batches_between_full_ones(rlk):
    T, H, V = 70, 256, 1000
    h, W, y = datagen.small_case(T, H, V, 132)
    lp = rlk.Logprob(H, V, entropy=True)
    hd, Wd, yd = dev_bits(h), dev_bits(W), dev_i32(y)
    say("one pass vs batches [0, 5, 0, 0, 33, 0, 32, 0] (x 1 and 4 vocab shards)")
    ref = lp.forward(hd, Wd, yd)
    sizes = [0, 5, 0, 0, 33, 0, 32, 0]
    for shards in (1, 4):
        o = lp.forward(hd, Wd, yd, batch_sizes=sizes, vocab_shards=shards)
        for k in ("logp", "lse", "entropy"):
            assert_bitwise(o[k], ref[k], f"{k} shards={shards}")
    want = oracle.logprob(h, W, y)["logp"]
    assert np.max(np.abs(host(ref["logp"]).astype(np.float64) - want)) <= 1e-3


def test_every_row_padded(rlk):
    T, H, V = 40, 256, 1000
    h, W, _ = datagen.small_case(T, H, V, 133)
    y = np.full(T, -1, dtype=np.int32)
    lp = rlk.Logprob(H, V, entropy=True)
    say("all 40 rows padded (targets = -1)")
    o = lp.forward(dev_bits(h), dev_bits(W), dev_i32(y), batch_sizes=[13, 27], vocab_shards=2)
    for k in ("logp", "lse", "entropy"):
        v = host(o[k])
        assert np.all(v.view(np.uint32) == 0), k  # +0.0 bit for bit
    assert lp.device_status(o["_workspace"]) == 0


@pytest.mark.parametrize("T", [1, 255, 257])
def test_single_row_and_ragged_row_tiles(rlk, T):
    """One row, and launches one row short of / past a 256-row tile: the rows past the end of
    the last row tile are clamped in the staging and never written."""
    import torch

    H, V = 256, 1000
    h, W, y = datagen.small_case(T, H, V, 134 + T)
    lp = rlk.Logprob(H, V)
    hd, Wd, yd = dev_bits(h), dev_bits(W), dev_i32(y)
    say(f"T = {T}: output buffers with guard words after the last row")
    guard = torch.full((T + 64,), float("nan"), dtype=torch.float32, device="cuda")
    out = {"logp": guard[:T], "lse": torch.empty(T, dtype=torch.float32, device="cuda")}
    o = lp.forward(hd, Wd, yd, out=out)
    torch.cuda.synchronize()
    assert np.all(np.isnan(host(guard[T:]))), "write past the last row"
    want = oracle.logprob(h, W, y)
    assert np.max(np.abs(host(o["logp"]).astype(np.float64) - want["logp"])) <= 1e-3
    assert np.max(np.abs(host(o["lse"]).astype(np.float64) - want["lse"])) <= 1e-3
    # the same rows one at a time
    one = lp.forward(hd, Wd, yd, batch_sizes=[1] * T) if T > 1 else o
    assert_bitwise(one["logp"], o["logp"], "logp row by row")
