"""The full-size workloads, in the launch configuration bench.py times (one pass) and in every
rollout/training layout they name. Parity against the float64 oracle is checked on every row,
against the oracle's outputs stored in tests/golden (reference_<workload>.npy, written by
make_reference.py from the oracle alone and tied to the input bytes by sha256), and on sampled
rows the oracle recomputes here; layout invariance on every row, byte for byte.
"""

import numpy as np
import pytest

import datagen
import oracle
from tests.helpers import (GOLDEN, assert_bitwise, dev_bits, dev_i32, diff_stats, golden_targets,
                           host, say)

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def head_inputs():
    w = datagen.WORKLOADS["qwen3_8b_head"]
    say("generating qwen3_8b_head inputs")
    h = datagen.hidden_bits(w)
    Wb = datagen.weight_bits(w)
    y, meta = golden_targets("qwen3_8b_head")
    assert meta["sha256_hidden"] == datagen.sha256(h) and meta["sha256_W"] == datagen.sha256(Wb)
    return w, h, Wb, y, dev_bits(h), dev_bits(Wb), dev_i32(y)


@pytest.fixture(scope="module")
def W64(head_inputs):
    return oracle.bf16_bits_to_f64(head_inputs[2])


def _reference(name, h, Wb, y, gamma=None):
    """The oracle's logp, lse and entropy of every row of a workload, stored with the sha256 of
    the inputs and targets they were computed from (checked here)."""
    import json
    import os

    ref = np.load(os.path.join(GOLDEN, f"reference_{name}.npy"), allow_pickle=False)
    with open(os.path.join(GOLDEN, f"reference_{name}.json")) as f:
        meta = json.load(f)
    assert meta["sha256_hidden"] == datagen.sha256(h), "reference belongs to other hidden bytes"
    assert meta["sha256_W"] == datagen.sha256(Wb), "reference belongs to another W"
    assert meta["sha256_targets"] == datagen.sha256(y), "reference belongs to other targets"
    if gamma is not None:
        assert meta["sha256_gamma"] == datagen.sha256(gamma)
    assert meta["sha256_values"] == datagen.sha256(ref)
    return {"logp": ref[0], "lse": ref[1], "entropy": ref[2]}


def _parity_all(got, ref, y, keys=("logp", "lse")):
    """Every active row within 1e-3 of the oracle; padded rows exactly +0.0. Prints the
    logprob_abs_diff_{mean,max,p50,p90,p99} report fields."""
    act = y >= 0
    for k in keys:
        s = diff_stats(got[k], ref[k], act)
        print(f"{k}: " + ", ".join(f"{k}_abs_diff_{q}={s[q]:.3e}"
                                     for q in ("mean", "max", "p50", "p90", "p99"))
              + f" over {s['n']} active rows", flush=True)
        assert s["max"] <= TOL, (k, s)
        assert np.all(got[k][~act] == 0.0) and not np.any(np.signbit(got[k][~act])), k


def _sample(n_rows, k, active):
    idx = np.nonzero(active)[0]
    return idx[np.linspace(0, idx.size - 1, k).astype(np.int64)]


def _parity(got, h, W64, y, rows, keys=("logp", "lse"), **kw):
    want = oracle.logprob(h, W64, y, rows=rows, want_entropy="entropy" in keys, **kw)
    for k in keys:
        s = diff_stats(got[k][rows], want[k])
        print(k, s, flush=True)
        assert s["max"] <= TOL, (k, s)


def test_qwen3_head_one_pass_matches_oracle_on_sampled_rows(rlk, head_inputs, W64):
    import torch

    w, h, Wb, y, hd, Wd, yd = head_inputs
    lp = rlk.Logprob(w.H, w.V, vocab_segments=4)
    say("qwen3_8b_head one pass")
    out = lp.forward(hd, Wd, yd)
    torch.cuda.synchronize()
    got = {k: host(out[k]) for k in ("logp", "lse")}
    assert np.all(got["logp"] <= 0.0) and np.all(np.isfinite(got["logp"]))
    _parity_all(got, _reference("qwen3_8b_head", h, Wb, y), y)
    _parity(got, h, W64, y, _sample(w.T, 32, y >= 0))


def test_qwen3_head_training_vs_rollout_layouts(rlk, head_inputs):
    import torch

    w, h, Wb, y, hd, Wd, yd = head_inputs
    lp = rlk.Logprob(w.H, w.V, vocab_segments=4)
    say("qwen3_8b_head reference (one pass)")
    ref = lp.forward(hd, Wd, yd)
    decode = datagen.decode_layout(w.T)
    for lay in (dict(row_chunk=1024), dict(row_chunk=2047), dict(batch_sizes=decode),
                dict(vocab_shards=2), dict(vocab_shards=4),
                dict(batch_sizes=decode, vocab_shards=2),
                dict(batch_sizes=decode, vocab_shards=4), dict(token_tile=128)):
        say(f"qwen3_8b_head layout {({k: (len(v) if k == 'batch_sizes' else v) for k, v in lay.items()})}")
        o = lp.forward(hd, Wd, yd, **lay)
        torch.cuda.synchronize()
        for k in ("logp", "lse"):
            assert_bitwise(o[k], ref[k], (k, str(lay)[:60]))


def test_qwen3_head_row_permutation(rlk, head_inputs):
    import torch

    w, h, Wb, y, hd, Wd, yd = head_inputs
    lp = rlk.Logprob(w.H, w.V, vocab_segments=4)
    perm = np.random.default_rng(11).permutation(w.T)
    say("qwen3_8b_head permuted rows")
    a = lp.forward(hd, Wd, yd)
    b = lp.forward(dev_bits(h[perm]), Wd, dev_i32(y[perm]))
    torch.cuda.synchronize()
    assert_bitwise(host(a["logp"])[perm], host(b["logp"]), "logp")


def test_qwen3_head_stress_hidden_x32(rlk, head_inputs, W64):
    """Parity-only stress input: the head's hidden scaled by 32 (exact in bf16), so the logits
    spread ~32x wider (sigma ~2.6 instead of ~0.08) and the tile maxima and EXP arguments cover
    a much larger range. Sampled oracle parity plus bitwise layouts."""
    import torch

    w, h, Wb, y, hd, Wd, yd = head_inputs
    def as_f32(bits):
        return (bits.astype(np.uint32) << 16).view(np.float32)

    f = as_f32(h) * np.float32(32.0)
    hs = datagen.f32_to_bf16_bits(f)
    assert np.array_equal(as_f32(hs), f)  # the scaling is exact
    hsd = dev_bits(hs)
    lp = rlk.Logprob(w.H, w.V, vocab_segments=4)
    say("stress x32: one pass")
    one = lp.forward(hsd, Wd, yd)
    torch.cuda.synchronize()
    got = {k: host(one[k]).copy() for k in ("logp", "lse")}
    for lay in (dict(row_chunk=1000), dict(vocab_shards=4)):
        say(f"stress x32: layout {lay}")
        o = lp.forward(hsd, Wd, yd, **lay)
        torch.cuda.synchronize()
        for k in ("logp", "lse"):
            assert_bitwise(o[k], one[k], (k, str(lay)))
    assert np.all(got["logp"] <= 0.0) and np.all(np.isfinite(got["logp"]))
    _parity(got, hs, W64, y, _sample(w.T, 24, y >= 0))


def test_tp4_shard_records_merge_equals_unsharded(rlk, head_inputs):
    import torch

    w, h, Wb, y, hd, Wd, yd = head_inputs
    lp = rlk.Logprob(w.H, w.V, vocab_segments=4)
    say("tp4: unsharded reference")
    ref = lp.forward(hd, Wd, yd)
    seg = w.V // 4
    recs = []
    for r in range(4):
        say(f"tp4: shard {r} partials")
        recs.append(lp.partials(hd, Wd[r * seg:(r + 1) * seg], r * seg, (r + 1) * seg, yd))
    say("tp4: merge")
    out = lp.merge(torch.cat(recs, 0).contiguous(), yd)
    torch.cuda.synchronize()
    for k in ("logp", "lse"):
        assert_bitwise(out[k], ref[k], k)


def test_long_grpo_chunkings_and_padding(rlk, head_inputs):
    import torch

    w = datagen.WORKLOADS["long_grpo"]
    Wb, Wd = head_inputs[2], head_inputs[5]
    say("generating long_grpo hidden")
    h = datagen.hidden_bits(w)
    y, meta = golden_targets("long_grpo")
    assert meta["sha256_hidden"] == datagen.sha256(h)
    pad = y < 0
    assert int(pad.sum()) == 553 and np.array_equal(pad, datagen.pad_mask(w))
    hd, yd = dev_bits(h), dev_i32(y)
    lp = rlk.Logprob(w.H, w.V, vocab_segments=4)
    say("long_grpo one pass")
    one = lp.forward(hd, Wd, yd)
    torch.cuda.synchronize()
    one_h = {k: host(one[k]).copy() for k in ("logp", "lse")}
    for k in one_h:
        v = one_h[k]
        assert np.all(v[pad] == 0.0) and not np.any(np.signbit(v[pad]))
        assert np.all(np.isfinite(v))
    for chunk in (8192, 2048):
        say(f"long_grpo chunks of {chunk}")
        o = lp.forward(hd, Wd, yd, row_chunk=chunk)
        torch.cuda.synchronize()
        for k in ("logp", "lse"):
            assert_bitwise(host(o[k]), one_h[k], (k, chunk))
    say("long_grpo with NaN hidden in padded rows")
    hn = hd.clone()
    hn[torch.from_numpy(np.nonzero(pad)[0]).cuda()] = -1  # bf16 NaN
    o = lp.forward(hn, Wd, yd, row_chunk=8192)
    torch.cuda.synchronize()
    for k in ("logp", "lse"):
        assert_bitwise(host(o[k]), one_h[k], (k, "nan pads"))
    del hn, hd
    _parity_all(one_h, _reference("long_grpo", h, Wb, y), y)
    W64 = oracle.bf16_bits_to_f64(Wb)
    _parity(one_h, h, W64, y, _sample(w.T, 16, ~pad))


def test_norm_head_one_pass_chunks_shards(rlk):
    import torch

    w = datagen.WORKLOADS["norm_head"]
    say("generating norm_head inputs")
    x = datagen.hidden_bits(w)
    Wb = datagen.weight_bits(w)
    g = datagen.gamma_bits(w)
    y, meta = golden_targets("norm_head")
    assert meta["sha256_W"] == datagen.sha256(Wb) and meta["sha256_gamma"] == datagen.sha256(g)
    xd, Wd, gd, yd = dev_bits(x), dev_bits(Wb), dev_bits(g), dev_i32(y)
    lp = rlk.Logprob(w.H, w.V, vocab_segments=4, temperature=w.tau, rmsnorm=True,
                     rms_eps=w.rms_eps, entropy=True)
    keys = ("logp", "lse", "entropy")
    say("norm_head one pass")
    one = lp.forward(xd, Wd, yd, gamma=gd)
    torch.cuda.synchronize()
    one_h = {k: host(one[k]).copy() for k in keys}
    for lay in (dict(row_chunk=2048), dict(vocab_shards=4), dict(row_chunk=2048, vocab_shards=4)):
        say(f"norm_head layout {lay}")
        o = lp.forward(xd, Wd, yd, gamma=gd, **lay)
        torch.cuda.synchronize()
        for k in keys:
            assert_bitwise(host(o[k]), one_h[k], (k, str(lay)))
    del xd
    _parity_all(one_h, _reference("norm_head", x, Wb, y, g), y, keys)
    W64 = oracle.bf16_bits_to_f64(Wb)
    rows = _sample(w.T, 16, y >= 0)
    _parity(one_h, x, W64, y, rows, keys, tau=w.tau, gamma_bits=g, rms_eps=w.rms_eps)
    assert np.all(one_h["entropy"] >= 0.0) and np.all(one_h["entropy"] <= np.log(w.V) + 1e-4)
