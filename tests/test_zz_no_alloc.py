"""rlk_logprob_forward_noalloc, the allocation-free forward (for callers that cannot allocate:
graph capture, serving loops), through the C ABI: bit for bit the outputs of
rlk_logprob_forward with a caller workspace, on two calls in a row (the second with fewer rows,
so the device scratch holds the first call's contents when the second starts), and a layout
whose workspace exceeds the scratch is refused before anything runs."""

import numpy as np
import pytest

import datagen
from invariant_lm_head_deterministic_amd import _lib
from tests.helpers import assert_bitwise, dev_bits, dev_i32, say

pytestmark = pytest.mark.gpu


def _call(rlk, lp, hd, Wd, yd, T, layout_kw, noalloc):
    import torch

    layout, keep = rlk.make_layout(T, **layout_kw)
    out = {k: torch.full((T,), 7.0, dtype=torch.float32, device="cuda")
           for k in ("logp", "lse", "entropy")}
    s = torch.cuda.current_stream().cuda_stream
    ent = out["entropy"].data_ptr() if lp.entropy else None
    if noalloc:
        _lib.rlk_logprob_forward_noalloc(lp.handle, hd.data_ptr(), Wd.data_ptr(), yd.data_ptr(),
                                         layout, None, out["logp"].data_ptr(),
                                         out["lse"].data_ptr(), ent, s)
    else:
        need = _lib.rlk_logprob_workspace_size(lp.config, layout)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        _lib.rlk_logprob_forward(lp.handle, hd.data_ptr(), Wd.data_ptr(), yd.data_ptr(), layout,
                                 None, out["logp"].data_ptr(), out["lse"].data_ptr(), ent,
                                 ws.data_ptr(), need, s)
    torch.cuda.synchronize()
    del keep
    return out


def test_noalloc_matches_forward_twice(rlk):
    w = datagen.WORKLOADS["qwen3_8b_head"]
    h, W = datagen.hidden_bits(w, rows=1024), datagen.weight_bits(w)
    y = np.load("tests/golden/targets_qwen3_8b_head.npy")[:1024].astype(np.int32)
    y[9::13] = -1
    hd, Wd, yd = dev_bits(h), dev_bits(W), dev_i32(y)
    lp = rlk.Logprob(w.H, w.V, vocab_segments=4, entropy=True)
    keys = ("logp", "lse", "entropy")
    # first call: 1024 rows as ragged decode batches over 4 shards (about 29 MB of workspace)
    sizes = datagen.decode_layout(1024)
    say(f"noalloc call 1: 1024 rows, {len(sizes)} batches x 4 shards")
    a = _call(rlk, lp, hd, Wd, yd, 1024, dict(batch_sizes=sizes, vocab_shards=4), True)
    b = _call(rlk, lp, hd, Wd, yd, 1024, dict(batch_sizes=sizes, vocab_shards=4), False)
    for k in keys:
        assert_bitwise(a[k], b[k], ("call 1", k))
    # second call: 77 rows in one pass, on a scratch that still holds the first call's data
    T2 = 77
    h2, y2 = hd[200:200 + T2].contiguous(), yd[200:200 + T2].contiguous()
    say("noalloc call 2: 77 rows, one pass")
    a2 = _call(rlk, lp, h2, Wd, y2, T2, {}, True)
    b2 = _call(rlk, lp, h2, Wd, y2, T2, {}, False)
    for k in keys:
        assert_bitwise(a2[k], b2[k], ("call 2", k))
    # and the same rows agree with the first call's (layout invariance through the scratch)
    for k in keys:
        assert_bitwise(a2[k], a[k][200:200 + T2], ("call 2 vs call 1", k))


def test_noalloc_refuses_more_than_its_scratch(rlk):
    w = datagen.WORKLOADS["qwen3_8b_head"]
    lp = rlk.Logprob(w.H, w.V, vocab_segments=4)
    T = 4096  # 78 MB of workspace at this vocabulary: more than the 64 MiB scratch
    layout, keep = rlk.make_layout(T)
    assert _lib.rlk_logprob_workspace_size(lp.config, layout) > 64 << 20
    with pytest.raises(_lib.RlkError) as e:
        # refused on the host before any pointer is used, so none is needed
        _lib.rlk_logprob_forward_noalloc(lp.handle, 16, 16, 16, layout, None, 16, 16, None, None)
    assert e.value.status == _lib.RLK_ERR_WORKSPACE
    del keep
