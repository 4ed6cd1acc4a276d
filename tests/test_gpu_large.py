"""Many rows: a hidden matrix of more than 2^32 bytes (2^21 + 3 rows of H = 1024), so that every
row, workspace and output offset needs 64-bit arithmetic. The one-pass result is compared with
row chunks bit for bit, and sampled rows (the first, the last, and rows around 2^20 and 2^21)
with the float64 oracle.

The GRPO run the pages report samples 8 responses per prompt of up to 6912 tokens (aihirek.info
report on the Qwen3-8B run); a rollout service batches far more rows than one such batch, and
the contract must not change with the row count (RL-Kernel v0.1.0 summary, "Numeric execution
contract").
"""

import numpy as np
import pytest

import datagen
import oracle
from tests.helpers import say

pytestmark = pytest.mark.gpu


def test_rows_past_2_to_32_bytes(rlk):
    import torch

    T, H, V = (1 << 21) + 3, 1024, 1000
    assert T * H * 2 > (1 << 32)
    say(f"T = {T}, H = {H}, V = {V}: generating hidden rows on the device")
    g = torch.Generator(device="cuda").manual_seed(151)
    hd = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    step = 1 << 18
    for r0 in range(0, T, step):
        r1 = min(T, r0 + step)
        hd[r0:r1] = torch.randn((r1 - r0, H), generator=g, device="cuda").to(torch.bfloat16)
    hd = hd.view(torch.int16)
    W = datagen.normal_bf16(V, H, 151, datagen.TID_W, scale=0.02)
    Wd = torch.from_numpy(W.view(np.int16)).cuda()
    yd = torch.randint(0, V, (T,), generator=g, device="cuda", dtype=torch.int32)
    yd[T - 2] = -1  # one padded row near the end
    lp = rlk.Logprob(H, V)
    say("one pass")
    a = lp.forward(hd, Wd, yd)
    la, sa = a["logp"].clone(), a["lse"].clone()
    del a
    say("row chunks of 2^20 + 5")
    b = lp.forward(hd, Wd, yd, row_chunk=(1 << 20) + 5)
    torch.cuda.synchronize()
    assert torch.equal(la.view(torch.int32), b["logp"].view(torch.int32))
    assert torch.equal(sa.view(torch.int32), b["lse"].view(torch.int32))
    del b
    rows = np.unique(np.array([0, 1, (1 << 20) - 1, 1 << 20, (1 << 20) + 1, (1 << 21) - 1,
                               1 << 21, T - 3, T - 2, T - 1]
                              + list(np.linspace(0, T - 1, 54).astype(np.int64))))
    idx = torch.from_numpy(rows).cuda()
    h_rows = hd.index_select(0, idx).cpu().numpy().view(np.uint16)
    y_rows = yd.index_select(0, idx).cpu().numpy()
    got = la.index_select(0, idx).cpu().numpy().astype(np.float64)
    got_lse = sa.index_select(0, idx).cpu().numpy().astype(np.float64)
    want = oracle.logprob(h_rows, W, y_rows)
    assert np.max(np.abs(got - want["logp"])) <= 1e-3
    assert np.max(np.abs(got_lse - want["lse"])) <= 1e-3
    pad = int(np.nonzero(rows == T - 2)[0][0])
    assert got[pad] == 0.0 and got_lse[pad] == 0.0
