"""The Python binding refuses malformed tensors before anything reaches the device: the C ABI
takes bare pointers, so a wrong shape, dtype, device or layout would otherwise become an
out-of-bounds access inside a kernel. No test here launches a kernel."""

import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def setup(rlk):
    import torch

    H, V, T = 256, 1000, 40
    dev = torch.device("cuda", 0)
    lp = rlk.Logprob(H, V, vocab_segments=4, rmsnorm=True, entropy=True)
    h = torch.zeros((T, H), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((V, H), dtype=torch.bfloat16, device=dev)
    y = torch.zeros(T, dtype=torch.int32, device=dev)
    g = torch.ones(H, dtype=torch.bfloat16, device=dev)
    return lp, h, W, y, g, dev


def test_forward_rejects_bad_tensors(setup):
    import torch

    lp, h, W, y, g, dev = setup
    bad = [
        dict(hidden=h[:, :128]),                        # wrong H (and not contiguous)
        dict(hidden=h[:39]),                            # fewer rows than targets
        dict(hidden=h.float()),                         # wrong dtype
        dict(hidden=h.cpu()),                           # wrong device
        dict(hidden=h.t().contiguous().t()),            # right shape, not contiguous
        dict(W=W[:999]),                                # wrong V
        dict(targets=y.long()),                         # wrong target dtype
        dict(targets=y.view(4, 10)),                    # not 1-D
        dict(gamma=g[:255]),                            # gamma shorter than H
        dict(out={"logp": torch.empty(39, device=dev), "lse": torch.empty(40, device=dev),
                  "entropy": torch.empty(40, device=dev)}),
        dict(workspace=torch.empty(10, dtype=torch.float32, device=dev)),
    ]
    for kw in bad:
        args = dict(hidden=h, W=W, targets=y, gamma=g)
        args.update(kw)
        hidden, Wx, targets = args.pop("hidden"), args.pop("W"), args.pop("targets")
        with pytest.raises((ValueError, TypeError)):
            lp.forward(hidden, Wx, targets, **args)


def test_partials_and_merge_reject_bad_tensors(setup):
    import torch

    lp, h, W, y, g, dev = setup
    seg = 250
    with pytest.raises(ValueError):
        lp.partials(h, W[:seg + 1], 0, seg, y, gamma=g)       # shard rows != vocab range
    with pytest.raises(ValueError):
        lp.partials(h[:30], W[:seg], 0, seg, y, gamma=g)      # hidden rows != targets
    with pytest.raises(ValueError):
        lp.partials(h, W[:seg], 0, seg, y, gamma=g,
                    records=torch.empty((1, 40, 3), device=dev))
    with pytest.raises(ValueError):
        lp.merge(torch.empty((3, 40, 4), device=dev), y)     # not all 4 segments
    with pytest.raises(ValueError):
        lp.merge(torch.empty((4, 40, 4), device=dev), y,
                 status=torch.empty(2, dtype=torch.int32, device=dev))
