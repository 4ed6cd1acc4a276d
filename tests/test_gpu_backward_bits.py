"""B1 (dz) bit for bit. dz lives only inside the backward, but with W the identity (V = H, one
segment) every logit is a hidden value exactly (one nonzero product per MFMA chain) and every dh
element is one dz element exactly (one nonzero term, the rest zeros), so dh exposes dz. In the
portable mode every step of B1 is an IEEE float32 operation or the software EXP, all of which the
float32 model of the contract (tests/contract_f32.py) reproduces; this pins the dz arithmetic and
its bf16 rounding (round to nearest even), including rows with a temperature and the entropy
gradient, rows whose probabilities underflow, and rows without a target (+0)."""

import numpy as np
import pytest

from tests import contract_f32 as cf
from tests.helpers import dev_bits, dev_i32, host, say

pytestmark = pytest.mark.gpu

F = np.float32


def _model_dh(h_bits, y, lse, g, gH, ent, inv_tau):
    """B1 in float32, then bf16: z' = z fl32(1/tau); p = EXP(z' - lse); d = 1 - p at the target
    else -p; q = g d; q -= gH (p ((z' - lse) + ent)); q *= fl32(1/tau); dz = bf16_rne(q)."""
    z = cf.bf16_to_f32(h_bits)
    with np.errstate(over="ignore", invalid="ignore"):  # rows without a target: lse = 0
        return _b1(z, y, lse, g, gH, ent, inv_tau)


def _b1(z, y, lse, g, gH, ent, inv_tau):
    temp = inv_tau != F(1.0)
    zp = z * inv_tau if temp else z
    x = zp - lse[:, None]
    p = cf.p_exp(x)
    V = z.shape[1]
    d = np.where(np.arange(V)[None, :] == y[:, None], F(1.0) - p, -p)
    q = g[:, None] * d
    if gH is not None:
        q = q - gH[:, None] * (p * (x + ent[:, None]))
    if temp:
        q = q * inv_tau
    dz = cf.bf16_to_f32(cf.f32_to_bf16_rne(q.astype(F)))
    dz[y < 0] = F(0.0)
    return dz


@pytest.mark.parametrize("tau,ent", [(1.0, False), (0.7, True)])
def test_dz_bits_match_the_float32_model(rlk, tau, ent):
    import torch

    T, H = 200, 512
    V = H
    rng = np.random.default_rng(4242)
    hf = rng.normal(scale=2.0, size=(T, H)).astype(F)
    hf[:8] *= F(40.0)  # wide rows: most probabilities underflow to 0 (and dz to a signed zero)
    h = cf.f32_to_bf16_rne(hf)
    W = np.zeros((V, H), dtype=np.uint16)
    W[np.arange(V), np.arange(V)] = 0x3F80  # bf16 1.0: W is the identity
    y = rng.integers(0, V, size=T).astype(np.int32)
    y[::9] = -1
    g = rng.normal(size=T).astype(F)
    gH = rng.normal(size=T).astype(F) if ent else None
    lp = rlk.Logprob(H, V, vocab_segments=1, temperature=tau, entropy=ent, portable=True)
    hd, Wd, yd = dev_bits(h), dev_bits(W), dev_i32(y)
    say(f"W = identity, T={T} H=V={H}, tau={tau}, entropy gradient={ent}")
    fw = lp.forward(hd, Wd, yd)
    gd = torch.from_numpy(g).cuda()
    gHd = None if gH is None else torch.from_numpy(gH).cuda()
    out = lp.backward(hd, Wd, yd, fw["lse"], gd, entropy=fw.get("entropy"), grad_entropy=gHd,
                      want_W=False)
    torch.cuda.synchronize()
    dh = host(out["grad_hidden"])
    lse = host(fw["lse"])
    e = host(fw["entropy"]) if ent else None
    inv_tau = F(lp.config.inv_temperature)
    want = _model_dh(h, y, lse, g, gH, e, inv_tau)
    # values compare as floats, so that +0 and -0 (a zero dz among zero terms) are equal
    bad = dh != want
    assert not np.any(bad), (int(bad.sum()), np.argwhere(bad)[:5].tolist())
    # and every nonzero element bit for bit
    nz = want != 0
    assert np.array_equal(dh[nz].view(np.uint32), want[nz].view(np.uint32))
    assert np.count_nonzero(want == 0) > 0 and np.count_nonzero(nz) > T * H // 2
