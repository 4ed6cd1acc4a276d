"""The backward (B1-B3) through the C ABI: parity with the float64 backward oracle, and bitwise
invariance of the gradients across row chunks, gradient accumulation and row order.

Parity bar, from the arithmetic: the one modelled rounding point is dz in bf16 (the oracle rounds
its float64 dz, the library its fp32 dz). The two roundings can land on neighbouring bf16 values
when the exact value sits near a rounding boundary, a difference of at most one bf16 step,
2^-7 |dz|; the fp32 MFMA chains add at most K/32 roundings of 2^-24 relative to the sum of
|terms|. So every element must satisfy
    |g_gpu - g_oracle| <= (2^-7 + 1e-4) (|dz| @ |W|)   for dh,  (|dz|^T @ |h|) for dW,
and the relative Frobenius error must stay under 1e-3 (flips are rare: it is ~1e-6 in practice).
"""

import numpy as np
import pytest

import datagen
import oracle
from tests.helpers import assert_bitwise, dev_bits, dev_i32, host, say

pytestmark = pytest.mark.gpu


def _inputs(T, H, V, cfg, pad_every=0):
    h, W, y = datagen.small_case(T, H, V, cfg)
    if pad_every:
        y[::pad_every] = -1
    g = np.random.default_rng(cfg).normal(size=T).astype(np.float32)
    gH = np.random.default_rng(cfg + 1).normal(size=T).astype(np.float32)
    return h, W, y, g, gH


def _run(rlk, h, W, y, g, gH=None, *, S=4, tau=1.0, portable=False, **kw):
    import torch

    T, H = h.shape
    V = W.shape[0]
    ent = gH is not None
    lp = rlk.Logprob(H, V, vocab_segments=S, temperature=tau, entropy=ent, portable=portable)
    hd, Wd, yd = dev_bits(h), dev_bits(W), dev_i32(y)
    fw = lp.forward(hd, Wd, yd)
    gd = torch.from_numpy(g).cuda()
    gHd = None if gH is None else torch.from_numpy(gH).cuda()
    out = lp.backward(hd, Wd, yd, fw["lse"], gd, entropy=fw.get("entropy"), grad_entropy=gHd,
                      **kw)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items() if not k.startswith("_")}, (lp, hd, Wd, yd, fw, gd,
                                                                            gHd)


def _abs_dz(h, W, y, g, gH, tau):
    hf = oracle.bf16_bits_to_f64(h)
    Wf = oracle.bf16_bits_to_f64(W)
    return np.abs(oracle.dlogits(hf @ Wf.T / tau, y, g, gH, tau))


def _check(got, h, W, y, g, gH, tau, rows_h=None, rows_w=None, dz=None):
    hf = oracle.bf16_bits_to_f64(h)
    Wf = oracle.bf16_bits_to_f64(W)
    want = oracle.grads(h, W, y, g, gH, tau=tau, dh_rows=rows_h, dW_rows=rows_w)
    dz = _abs_dz(h, W, y, g, gH, tau) if dz is None else dz
    rh = np.arange(h.shape[0]) if rows_h is None else rows_h
    rw = np.arange(W.shape[0]) if rows_w is None else rows_w
    for key, ref, bound in (("grad_hidden", want["dh"], dz[rh] @ np.abs(Wf)),
                            ("grad_W", want["dW"], dz[:, rw].T @ np.abs(hf))):
        gg = got[key][rh] if key == "grad_hidden" else got[key][rw]
        d = np.abs(gg.astype(np.float64) - ref)
        lim = (2.0 ** -7 + 1e-4) * bound + 1e-30
        fro = np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)
        print(key, "max", float(d.max()), "max/lim", float((d / lim).max()), "fro", fro, flush=True)
        assert np.all(d <= lim), (key, float((d / lim).max()))
        assert fro <= 1e-3, (key, fro)


def _check_exact(got, h, W, y, g, gH, tau, rows_h=None, rows_w=None, dz=None):
    """Against the exact gradient (the oracle without its bf16 dz boundary). The library rounds
    its fp32 dz to bf16 once, an error of at most half a bf16 step, 2^-8 |dz| (8 significant
    bits); its fp32 dz differs from the exact one by ~1e-6 relative and the fp32 MFMA chains add
    ~K/32 roundings of 2^-24. So every element must satisfy
        |g_gpu - g_exact| <= (2^-8 + 1e-4) (|dz| @ |W|)   (dh),   (|dz|^T @ |h|)   (dW).
    The relative Frobenius error is printed: it is what the bf16 boundary costs the gradient."""
    hf = oracle.bf16_bits_to_f64(h)
    Wf = oracle.bf16_bits_to_f64(W)
    want = oracle.grads(h, W, y, g, gH, tau=tau, round_dz=False, dh_rows=rows_h, dW_rows=rows_w)
    dz = _abs_dz(h, W, y, g, gH, tau) if dz is None else dz
    rh = np.arange(h.shape[0]) if rows_h is None else rows_h
    rw = np.arange(W.shape[0]) if rows_w is None else rows_w
    out = {}
    for key, ref, bound in (("grad_hidden", want["dh"], dz[rh] @ np.abs(Wf)),
                            ("grad_W", want["dW"], dz[:, rw].T @ np.abs(hf))):
        gg = got[key][rh] if key == "grad_hidden" else got[key][rw]
        d = np.abs(gg.astype(np.float64) - ref)
        lim = (2.0 ** -8 + 1e-4) * bound + 1e-30
        fro = np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)
        print(key, "vs exact: max", float(d.max()), "max/lim", float((d / lim).max()),
              "rel fro", fro, flush=True)
        assert np.all(d <= lim), (key, float((d / lim).max()))
        out[key] = fro
    return out


CASES = [
    # T, H, V, S_c, tau, entropy gradient, pad every
    (300, 256, 5000, 4, 1.0, False, 0),   # 3 row tiles, segments of 1250 (Lp 1280)
    (77, 384, 3000, 2, 0.7, True, 5),     # temperature, entropy gradient, padded rows
    (33, 128, 1000, 1, 1.0, True, 0),     # one segment: no tree
    (130, 256, 5600, 8, 1.0, False, 7),   # 8 segments of 700 (Lp 768)
    (1, 128, 1000, 4, 1.0, False, 0),     # a single row, segments of 250 (not a multiple of 4)
]


@pytest.mark.parametrize("T,H,V,S,tau,ent,pad", CASES)
def test_backward_matches_oracle(rlk, T, H, V, S, tau, ent, pad):
    h, W, y, g, gH = _inputs(T, H, V, 500 + T, pad)
    say(f"backward T={T} H={H} V={V} S={S} tau={tau} ent={ent}")
    got, _ = _run(rlk, h, W, y, g, gH if ent else None, S=S, tau=tau)
    dz = _abs_dz(h, W, y, g, gH if ent else None, tau)
    _check(got, h, W, y, g, gH if ent else None, tau, dz=dz)
    _check_exact(got, h, W, y, g, gH if ent else None, tau, dz=dz)


def test_backward_portable_matches_oracle(rlk):
    T, H, V = 150, 256, 3000
    h, W, y, g, gH = _inputs(T, H, V, 520, 9)
    say("backward portable")
    got, _ = _run(rlk, h, W, y, g, gH, S=4, tau=0.8, portable=True)
    _check(got, h, W, y, g, gH, 0.8)


def test_backward_chunks_accumulation_and_order_are_bitwise_invariant(rlk):
    import torch

    T, H, V = 300, 256, 4000
    h, W, y, g, gH = _inputs(T, H, V, 530, 11)
    say("backward invariances")
    one, (lp, hd, Wd, yd, fw, gd, gHd) = _run(rlk, h, W, y, g, gH, S=4)
    ent = fw["entropy"]
    for rc in (128, 256):
        o = lp.backward(hd, Wd, yd, fw["lse"], gd, entropy=ent, grad_entropy=gHd, row_chunk=rc)
        torch.cuda.synchronize()
        assert_bitwise(o["grad_hidden"], one["grad_hidden"], f"dh chunk {rc}")
        assert_bitwise(o["grad_W"], one["grad_W"], f"dW chunk {rc}")
    # two micro-batches: rows [0, 256) then [256, 300) accumulated into the same grad_W
    gw = torch.empty((V, H), dtype=torch.float32, device="cuda")
    a = lp.backward(hd[:256].contiguous(), Wd, yd[:256].contiguous(), fw["lse"][:256].contiguous(),
                    gd[:256].contiguous(), entropy=ent[:256].contiguous(),
                    grad_entropy=gHd[:256].contiguous(), grad_W=gw)
    b = lp.backward(hd[256:].contiguous(), Wd, yd[256:].contiguous(), fw["lse"][256:].contiguous(),
                    gd[256:].contiguous(), entropy=ent[256:].contiguous(),
                    grad_entropy=gHd[256:].contiguous(), grad_W=gw, accumulate=True)
    torch.cuda.synchronize()
    assert_bitwise(gw, one["grad_W"], "dW accumulated")
    assert_bitwise(torch.cat([a["grad_hidden"], b["grad_hidden"]]), one["grad_hidden"], "dh split")
    # rows are independent in dh: a permutation permutes it
    perm = np.random.default_rng(4).permutation(T)
    pt = torch.from_numpy(perm).cuda()
    o = lp.backward(hd[pt].contiguous(), Wd, yd[pt].contiguous(), fw["lse"][pt].contiguous(),
                    gd[pt].contiguous(), entropy=ent[pt].contiguous(),
                    grad_entropy=gHd[pt].contiguous(), want_W=False)
    torch.cuda.synchronize()
    assert_bitwise(host(o["grad_hidden"]), one["grad_hidden"][perm], "dh permuted")
    # run to run
    o = lp.backward(hd, Wd, yd, fw["lse"], gd, entropy=ent, grad_entropy=gHd)
    torch.cuda.synchronize()
    assert_bitwise(o["grad_hidden"], one["grad_hidden"], "dh repeat")
    assert_bitwise(o["grad_W"], one["grad_W"], "dW repeat")


def test_backward_only_one_gradient(rlk):
    T, H, V = 64, 128, 1000
    h, W, y, g, _ = _inputs(T, H, V, 540)
    say("backward single outputs")
    both, (lp, hd, Wd, yd, fw, gd, _) = _run(rlk, h, W, y, g)
    import torch

    oh = lp.backward(hd, Wd, yd, fw["lse"], gd, want_W=False)
    ow = lp.backward(hd, Wd, yd, fw["lse"], gd, want_hidden=False)
    torch.cuda.synchronize()
    assert "grad_W" not in oh and "grad_hidden" not in ow
    assert_bitwise(oh["grad_hidden"], both["grad_hidden"], "dh alone")
    assert_bitwise(ow["grad_W"], both["grad_W"], "dW alone")


def test_backward_refusals(rlk):
    import torch

    H, V = 128, 1000
    h, W, y, g, gH = _inputs(8, H, V, 550)
    hd, Wd, yd = dev_bits(h), dev_bits(W), dev_i32(y)
    lse = torch.zeros(8, dtype=torch.float32, device="cuda")
    gd = torch.from_numpy(g).cuda()
    lp = rlk.Logprob(H, V, rmsnorm=True)
    with pytest.raises(rlk.RlkError):  # the RMSNorm's gamma is required
        lp.backward(hd, Wd, yd, lse, gd)
    lp = rlk.Logprob(H, V)  # no entropy flag
    with pytest.raises(rlk.RlkError):
        lp.backward(hd, Wd, yd, lse, gd, entropy=lse, grad_entropy=torch.from_numpy(gH).cuda())
    with pytest.raises(rlk.RlkError):
        lp.backward(hd, Wd, yd, lse, gd, row_chunk=100)
    with pytest.raises(ValueError):
        lp.backward(hd, Wd, yd, lse[:4], gd)
    lp4 = rlk.Logprob(H, V, vocab_segments=4)
    with pytest.raises(rlk.RlkError):  # a shard must be whole segments (of 250 here)
        lp4.backward_partials(hd, Wd[:300].contiguous(), 0, 300, yd, lse, gd)
    with pytest.raises(ValueError):  # the merge takes every segment's partial
        lp4.backward_merge(torch.zeros((2, 8, H), dtype=torch.float32, device="cuda"))


def test_backward_full_size_sampled(rlk):
    """Qwen3-8B head shape (T=4096, H=4096, V=151936, 4 segments): sampled rows of dh and of dW
    against the oracle (which still reduces over every row and every vocab index)."""
    w = datagen.WORKLOADS["qwen3_8b_head"]
    h, W = datagen.hidden_bits(w), datagen.weight_bits(w)
    y = np.load("tests/golden/targets_qwen3_8b_head.npy").astype(np.int32)
    g = np.random.default_rng(560).normal(size=w.T).astype(np.float32)
    say("backward full size")
    got, _ = _run(rlk, h, W, y, g, S=w.segments)
    rows_h = np.array([0, 1, 777, 2048, 4095])
    rows_w = np.concatenate([y[[0, 777]], [0, 37983, 37984, 75968, 151935]])
    dz = _abs_dz(h, W, y, g, None, 1.0)
    _check(got, h, W, y, g, None, 1.0, rows_h=rows_h, rows_w=rows_w, dz=dz)
    _check_exact(got, h, W, y, g, None, 1.0, rows_h=rows_h, rows_w=rows_w, dz=dz)


def _rms_inputs(T, H, V, cfg, pad_every=0):
    x = datagen.normal_bf16(T, H, cfg, datagen.TID_HIDDEN)
    W = datagen.normal_bf16(V, H, cfg, datagen.TID_W, scale=0.02)
    gam = datagen.normal_bf16(1, H, cfg, datagen.TID_GAMMA, scale=0.1, mean=1.0)[0]
    y = datagen.uniform_targets(T, V, cfg)
    if pad_every:
        y[::pad_every] = -1
    g = np.random.default_rng(cfg).normal(size=T).astype(np.float32)
    gH = np.random.default_rng(cfg + 1).normal(size=T).astype(np.float32)
    return x, W, gam, y, g, gH


def _run_rms(rlk, x, W, gam, y, g, gH, *, S, tau, eps=1e-6, **kw):
    import torch

    T, H = x.shape
    V = W.shape[0]
    lp = rlk.Logprob(H, V, vocab_segments=S, temperature=tau, rmsnorm=True, rms_eps=eps,
                     entropy=gH is not None)
    xd, Wd, yd, gd_ = dev_bits(x), dev_bits(W), dev_i32(y), dev_bits(gam)
    fw = lp.forward(xd, Wd, yd, gamma=gd_)
    gd = torch.from_numpy(g).cuda()
    gHd = None if gH is None else torch.from_numpy(gH).cuda()
    out = lp.backward(xd, Wd, yd, fw["lse"], gd, entropy=fw.get("entropy"), grad_entropy=gHd,
                      gamma=gd_, **kw)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items() if not k.startswith("_")}, (lp, xd, Wd, yd, gd_, fw,
                                                                            gd, gHd)


def _rel(got, ref):
    d = np.abs(got.astype(np.float64) - ref)
    return float(d.max() / max(np.abs(ref).max(), 1e-300)), \
        float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))


@pytest.mark.parametrize("T,H,V,S,tau,ent", [
    (200, 256, 3000, 4, 0.7, True),
    (90, 384, 2000, 2, 1.0, False),
])
def test_backward_rmsnorm_matches_oracle(rlk, T, H, V, S, tau, ent):
    """Through the RMSNorm, on top of the dz flips of the plain backward, the bf16 rounding of y
    may land one step apart in the fp32 and fp64 RMSNorms (rarely), and r is an fp32 reciprocal
    square root (~1e-7 relative). grad_W = dz^T y then moves by at most one bf16 step of dz or of
    y per term: |err| <= 2^-6 (|dz|^T @ |y|) per element. grad_hidden and grad_gamma mix every
    element of a row, so their bar is relative: max error <= 1e-3 of the largest element and a
    relative Frobenius error <= 1e-4."""
    x, W, gam, y, g, gH = _rms_inputs(T, H, V, 600 + T, 7)
    gH = gH if ent else None
    say(f"backward rmsnorm T={T} H={H} V={V} S={S} tau={tau} ent={ent}")
    got, _ = _run_rms(rlk, x, W, gam, y, g, gH, S=S, tau=tau)
    want = oracle.grads(x, W, y, g, gH, tau=tau, gamma_bits=gam, rms_eps=1e-6)
    for key, ref in (("grad_hidden", want["dh"]), ("grad_gamma", want["dgamma"])):
        mx, fro = _rel(got[key], ref)
        print(key, "max/maxref", mx, "fro", fro, flush=True)
        assert mx <= 1e-3 and fro <= 1e-4, (key, mx, fro)
    yn = oracle.rmsnorm_bf16(oracle.bf16_bits_to_f64(x), oracle.bf16_bits_to_f64(gam), 1e-6)
    dz = np.abs(oracle.dlogits(yn @ oracle.bf16_bits_to_f64(W).T / tau, y, g, gH, tau))
    lim = 2.0 ** -6 * (dz.T @ np.abs(yn)) + 1e-30
    d = np.abs(got["grad_W"].astype(np.float64) - want["dW"])
    print("grad_W max/lim", float((d / lim).max()), "fro", _rel(got["grad_W"], want["dW"])[1],
          flush=True)
    assert np.all(d <= lim)
    assert _rel(got["grad_W"], want["dW"])[1] <= 1e-3


def test_backward_rmsnorm_chunks_and_accumulation_bitwise(rlk):
    import torch

    T, H, V = 300, 256, 2500
    x, W, gam, y, g, gH = _rms_inputs(T, H, V, 610, 13)
    say("backward rmsnorm invariances")
    one, (lp, xd, Wd, yd, gd_, fw, gd, gHd) = _run_rms(rlk, x, W, gam, y, g, gH, S=4, tau=1.0)
    ent = fw["entropy"]
    o = lp.backward(xd, Wd, yd, fw["lse"], gd, entropy=ent, grad_entropy=gHd, gamma=gd_,
                    row_chunk=128)
    torch.cuda.synchronize()
    for k in ("grad_hidden", "grad_W", "grad_gamma"):
        assert_bitwise(o[k], one[k], f"{k} chunk 128")
    gw = torch.empty((V, H), dtype=torch.float32, device="cuda")
    gg = torch.empty((H,), dtype=torch.float32, device="cuda")
    sl = [slice(0, 256), slice(256, T)]
    for i, s_ in enumerate(sl):
        lp.backward(xd[s_].contiguous(), Wd, yd[s_].contiguous(), fw["lse"][s_].contiguous(),
                    gd[s_].contiguous(), entropy=ent[s_].contiguous(),
                    grad_entropy=gHd[s_].contiguous(), gamma=gd_, want_hidden=False, grad_W=gw,
                    grad_gamma=gg, accumulate=i > 0)
    torch.cuda.synchronize()
    assert_bitwise(gw, one["grad_W"], "dW accumulated")
    assert_bitwise(gg, one["grad_gamma"], "dgamma accumulated")


def test_backward_norm_head_rows_full_width(rlk):
    """norm_head's widths (H=5120, V=151936, tau=0.7, entropy) on its first 512 rows."""
    w = datagen.WORKLOADS["norm_head"]
    T = 512
    x = datagen.hidden_bits(w, rows=T)
    W = datagen.weight_bits(w)
    gam = datagen.gamma_bits(w)
    y = np.load("tests/golden/targets_norm_head.npy")[:T].astype(np.int32)
    g = np.random.default_rng(620).normal(size=T).astype(np.float32)
    gH = np.random.default_rng(621).normal(size=T).astype(np.float32)
    say("backward norm_head 512 rows")
    got, _ = _run_rms(rlk, x, W, gam, y, g, gH, S=w.segments, tau=w.tau, eps=w.rms_eps)
    want = oracle.grads(x, W, y, g, gH, tau=w.tau, gamma_bits=gam, rms_eps=w.rms_eps,
                        dW_rows=np.concatenate([y[:3], [0, 151935]]))
    mx, fro = _rel(got["grad_hidden"], want["dh"])
    print("grad_hidden", mx, fro, flush=True)
    assert mx <= 1e-3 and fro <= 1e-4
    mx, fro = _rel(got["grad_gamma"], want["dgamma"])
    print("grad_gamma", mx, fro, flush=True)
    assert mx <= 1e-3 and fro <= 1e-4
    rw = np.concatenate([y[:3], [0, 151935]])
    mx, fro = _rel(got["grad_W"][rw], want["dW"])
    print("grad_W", mx, fro, flush=True)
    assert mx <= 1e-3 and fro <= 1e-4


@pytest.mark.parametrize("rms", [False, True])
def test_backward_vocab_shards_equal_one_pass(rlk, rms):
    """Shards of 1, 2 and 4 segments (S_c = 4) computing their dh partials and grad_W rows, merged
    in the segment tree, give the one-pass backward's bits: the vocab-parallel split of B2/B3."""
    import torch

    T, H, V, S = 200, 256, 3000, 4
    if rms:
        x, W, gam, y, g, gH = _rms_inputs(T, H, V, 640, 9)
        one, (lp, xd, Wd, yd, gd_, fw, gd, gHd) = _run_rms(rlk, x, W, gam, y, g, gH, S=S,
                                                            tau=0.7)
    else:
        h, W, y, g, gH = _inputs(T, H, V, 650, 9)
        one, (lp, xd, Wd, yd, fw, gd, gHd) = _run(rlk, h, W, y, g, gH, S=S, tau=0.7)
        gd_ = None
    ent = fw["entropy"]
    seg = V // S
    for cuts in ([0, 4], [0, 2, 4], [0, 1, 2, 3, 4], [0, 1, 4]):
        say(f"backward shards {cuts} rms={rms}")
        parts, rows = [], []
        for a, b in zip(cuts[:-1], cuts[1:]):
            v0, v1 = a * seg, b * seg
            o = lp.backward_partials(xd, Wd[v0:v1].contiguous(), v0, v1, yd, fw["lse"], gd,
                                     entropy=ent, grad_entropy=gHd, gamma=gd_)
            parts.append(o["dh_parts"])
            rows.append(o["grad_W_shard"])
        m = lp.backward_merge(torch.cat(parts), hidden=xd if rms else None, gamma=gd_)
        torch.cuda.synchronize()
        assert_bitwise(m["grad_hidden"], one["grad_hidden"], f"dh {cuts}")
        assert_bitwise(torch.cat(rows), one["grad_W"], f"dW {cuts}")
        if rms:
            assert_bitwise(m["grad_gamma"], one["grad_gamma"], f"dgamma {cuts}")
