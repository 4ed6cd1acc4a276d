"""The forward and the backward captured in a HIP graph and replayed.

A rollout engine replays its decode step from a captured graph, so the recompute path has to be
capturable: no allocation, no memset node, no host synchronization inside a call. The persistent
LM-head kernel's work-queue counters are zeroed by a kernel at the start of every forward and
reset by the kernel's last block, so every replay starts from zero. Each replay is checked bit
for bit against the eager result, with other eager work on the same device in between.
"""

import numpy as np
import pytest

import datagen
from tests.helpers import assert_bitwise, dev_bits, dev_i32, host, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize(
    "layout", [dict(), dict(batch_sizes=[1, 255, 0, 20, 40, 100, 284], vocab_shards=4)])
def test_forward_graph_replays_equal_eager(rlk, layout):
    import torch

    T, H, V = 700, 512, 4000
    h, W, y = datagen.small_case(T, H, V, 141)
    h2, _, y2 = datagen.small_case(T, H, V, 142)
    lp = rlk.Logprob(H, V, entropy=True)
    hd, Wd, yd = dev_bits(h), dev_bits(W), dev_i32(y)
    h2d, y2d = dev_bits(h2), dev_i32(y2)
    say(f"eager forward, layout {layout}")
    ref = lp.forward(hd, Wd, yd, **layout)
    other = lp.forward(h2d, Wd, y2d)
    torch.cuda.synchronize()
    ref = {k: host(ref[k]).copy() for k in ("logp", "lse", "entropy")}
    other = {k: host(other[k]).copy() for k in ("logp", "lse", "entropy")}

    ws = torch.empty(lp.workspace_size(T, **layout), dtype=torch.uint8, device="cuda")
    out = {k: torch.empty(T, dtype=torch.float32, device="cuda") for k in ("logp", "lse", "entropy")}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lp.forward(hd, Wd, yd, workspace=ws, out=out, **layout)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    say("capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lp.forward(hd, Wd, yd, workspace=ws, out=out, **layout)
    for rep in range(4):
        say(f"replay {rep}")
        for v in out.values():
            v.fill_(float("nan"))
        # eager work of the program between replays, on the same workspace-free path
        e = lp.forward(h2d, Wd, y2d)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ("logp", "lse", "entropy"):
            assert_bitwise(host(out[k]), ref[k], f"replay {rep} {k}")
            assert_bitwise(host(e[k]), other[k], f"eager between replays {k}")
        assert lp.device_status(ws) == 0


def test_backward_graph_replays_equal_eager(rlk):
    import torch

    T, H, V = 384, 256, 2000
    h, W, y = datagen.small_case(T, H, V, 143)
    lp = rlk.Logprob(H, V)
    hd, Wd, yd = dev_bits(h), dev_bits(W), dev_i32(y)
    gl = torch.from_numpy(np.random.default_rng(143).normal(size=T).astype(np.float32)).cuda()
    say("eager backward")
    f = lp.forward(hd, Wd, yd)
    lse = f["lse"].clone()
    ref = lp.backward(hd, Wd, yd, lse, gl)
    torch.cuda.synchronize()
    ref = {k: host(ref[k]).copy() for k in ("grad_hidden", "grad_W")}

    wsb = torch.empty(rlk.rlk_logprob_backward_workspace_size(lp.config, T, 0), dtype=torch.uint8,
                      device="cuda")
    gW = torch.empty((V, H), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lp.backward(hd, Wd, yd, lse, gl, grad_W=gW, workspace=wsb)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    say("capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        o = lp.backward(hd, Wd, yd, lse, gl, grad_W=gW, workspace=wsb)
    for rep in range(3):
        say(f"replay {rep}")
        gW.fill_(float("nan"))
        o["grad_hidden"].fill_(float("nan"))
        lp.forward(hd, Wd, yd)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_bitwise(host(gW), ref["grad_W"], f"replay {rep} grad_W")
        assert_bitwise(host(o["grad_hidden"]), ref["grad_hidden"], f"replay {rep} grad_hidden")
