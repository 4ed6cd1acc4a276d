"""Calls enqueued on a side stream (not torch's current one): the binding's own allocations
(workspace, records, outputs) are recorded on that stream, so the caching allocator cannot hand
them out while the kernels still use them. Results equal the default-stream run bit for bit,
also when other allocations churn the allocator between enqueue and synchronization."""

import numpy as np
import pytest

import datagen
from tests.helpers import assert_bitwise, dev_bits, dev_i32, say

pytestmark = pytest.mark.gpu


def test_side_stream_partials_merge_forward(rlk):
    import torch

    T, H, V, S = 300, 512, 8000, 4
    h, W, y = datagen.small_case(T, H, V, 611)
    hd, Wd, yd = dev_bits(h), dev_bits(W), dev_i32(y)
    lp = rlk.Logprob(H, V, vocab_segments=S, entropy=True)
    seg = V // S
    say("default stream reference")
    ref = lp.forward(hd, Wd, yd)
    ref_rec = torch.cat([lp.partials(hd, Wd[r * seg:(r + 1) * seg], r * seg, (r + 1) * seg, yd)
                         for r in range(S)]).contiguous()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    say("side stream: partials, merge, forward, with allocator churn on the current stream")
    recs = []
    for r in range(S):
        recs.append(lp.partials(hd, Wd[r * seg:(r + 1) * seg], r * seg, (r + 1) * seg, yd,
                                stream=side))
        # churn: allocations on the current stream that could reuse freed blocks
        junk = [torch.full((1 << 20,), 3.0, device="cuda") for _ in range(4)]
        del junk
    with torch.cuda.stream(side):
        cat = torch.cat(recs).contiguous()
    mg = lp.merge(cat, yd, stream=side)
    fw = lp.forward(hd, Wd, yd, stream=side)
    junk = [torch.full((1 << 22,), -1.0, device="cuda") for _ in range(4)]
    del junk
    side.synchronize()
    torch.cuda.synchronize()
    assert_bitwise(cat, ref_rec, "records")
    for k in ("logp", "lse", "entropy"):
        assert_bitwise(mg[k], ref[k], ("merge", k))
        assert_bitwise(fw[k], ref[k], ("forward", k))
