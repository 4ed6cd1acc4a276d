"""The persistent kernels hand out their items through work queues, so which CU computes which
tile changes from run to run with the CUs' clocks and whatever else occupies the device. The
results must not change with it: the forward (LM-head kernel with its queues, fused fold) and the
backward (persistent dz, dh and dW GEMMs) are run while a side stream keeps large matrix products
in flight on the same GPU, which takes CUs away from the library's blocks at varying moments, and
every output is compared bit for bit with the run on an otherwise idle device."""

import numpy as np
import pytest

import datagen
from tests.helpers import assert_bitwise, dev_bits, dev_i32, say

pytestmark = pytest.mark.gpu


def _load(torch, side, n):
    """n fp32 matrix products of 4096^3 (~1 ms each) enqueued on `side` (plain 2-D operands)."""
    a = torch.randn(4096, 4096, device="cuda")
    b = torch.randn(4096, 4096, device="cuda")
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(n):
            a = torch.mm(a, b) * 1e-2
    return a


def test_forward_and_backward_bits_under_concurrent_load(rlk):
    import torch

    T, H, V, S = 1100, 512, 24000, 4  # 5 row tiles x 92 vocab blocks: many queue items
    h, W, y = datagen.small_case(T, H, V, 907)
    hd, Wd, yd = dev_bits(h), dev_bits(W), dev_i32(y)
    g = torch.from_numpy(np.random.default_rng(907).normal(size=T).astype(np.float32)).cuda()
    lp = rlk.Logprob(H, V, vocab_segments=S, entropy=True)
    say("reference on an idle device (after a warm-up call)")
    lp.backward(hd, Wd, yd, lp.forward(hd, Wd, yd)["lse"], g)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    ref = lp.forward(hd, Wd, yd)
    ref_b = lp.backward(hd, Wd, yd, ref["lse"], g)
    e1.record()
    torch.cuda.synchronize()
    idle_ms = e0.elapsed_time(e1)
    side = torch.cuda.Stream()  # default priority
    for rep in range(3):
        say(f"under load, repeat {rep}")
        keep = _load(torch, side, 6 + 4 * rep)
        e0.record()
        o = lp.forward(hd, Wd, yd)
        ob = lp.backward(hd, Wd, yd, o["lse"], g)
        e1.record()
        torch.cuda.synchronize()
        del keep
        # how much the load slowed the library's calls (printed: evidence of the overlap)
        say(f"forward + backward: {e0.elapsed_time(e1):.3f} ms under load, {idle_ms:.3f} ms idle")
        for k in ("logp", "lse", "entropy"):
            assert_bitwise(o[k], ref[k], f"{k} (repeat {rep})")
        for k in ("grad_hidden", "grad_W"):
            assert_bitwise(ob[k], ref_b[k], f"{k} (repeat {rep})")
