"""Pins of the float32 contract model (tests/contract_f32.py) that the portable GPU mode is
checked against bit for bit: its software EXP, LOG and RSQ against float64 libm within stated ulp
bounds and at their special values; its tree order on a case where order decides the result; and
the whole model against the float64 oracle."""

import numpy as np
import pytest

import datagen
import oracle
from tests import contract_f32 as cf


def _ulps(got: np.ndarray, exact: np.ndarray) -> np.ndarray:
    """|got - exact| in units of the fp32 spacing at the exact value (subnormal spacing 2^-149)."""
    sp = np.maximum(np.spacing(np.abs(exact.astype(np.float32))).astype(np.float64), 2.0 ** -149)
    return np.abs(got.astype(np.float64) - exact) / sp


def _bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def test_p_exp_within_1p25_ulp():
    g = np.random.default_rng(11)
    x = np.concatenate([g.uniform(-103.97, 88.72, 600_000), g.uniform(-30.0, 0.0, 300_000),
                        g.uniform(-1.0, 1.0, 100_000),
                        g.uniform(-103.97, -87.34, 100_000)]).astype(np.float32)  # subnormal out
    e = _ulps(cf.p_exp(x), np.exp(x.astype(np.float64)))
    assert e.max() <= 1.25, (e.max(), x[e.argmax()])
    assert np.mean(e > 0.5) < 0.15  # mostly correctly rounded


def test_p_exp_special_values():
    assert _bits(cf.p_exp(np.float32(0.0))) == _bits(1.0)
    assert _bits(cf.p_exp(np.float32(-0.0))) == _bits(1.0)
    assert _bits(cf.p_exp(np.float32(-np.inf))) == _bits(0.0)
    assert cf.p_exp(np.float32(np.inf)) == np.inf
    assert np.isnan(cf.p_exp(np.float32(np.nan)))
    assert cf.p_exp(np.float32(89.0)) == np.inf
    assert _bits(cf.p_exp(np.float32(-104.0))) == _bits(0.0)
    top = np.nextafter(np.float32(88.72283), np.float32(0))
    assert np.isfinite(cf.p_exp(top)) and cf.p_exp(top) > 3.0e38
    # e^(ln 2^-149) is the smallest subnormal; e^(-149.5 ln 2) rounds to it or to 2^-150 -> 0
    assert cf.p_exp(np.float32(-149 * np.log(2.0))) == np.float32(2.0 ** -149)
    # exact powers of e^1 against libm
    k = np.arange(-80, 81, dtype=np.float32)
    assert _ulps(cf.p_exp(k), np.exp(k.astype(np.float64))).max() <= 1.25


def test_p_log_within_1_ulp():
    g = np.random.default_rng(12)
    b = g.integers(1, 0x7F800000, 600_000, dtype=np.uint32).view(np.float32)  # incl. subnormals
    near1 = (1.0 + g.uniform(-0.3, 0.42, 300_000)).astype(np.float32)
    x = np.concatenate([b, near1])
    e = _ulps(cf.p_log(x), np.log(x.astype(np.float64)))
    assert e.max() <= 1.0, (e.max(), x[e.argmax()])


def test_p_log_special_values():
    assert _bits(cf.p_log(np.float32(1.0))) == _bits(0.0)
    assert cf.p_log(np.float32(0.0)) == -np.inf
    assert cf.p_log(np.float32(-0.0)) == -np.inf
    assert np.isnan(cf.p_log(np.float32(-1.0)))
    assert np.isnan(cf.p_log(np.float32(np.nan)))
    assert cf.p_log(np.float32(np.inf)) == np.inf
    k = np.arange(-149, 128)
    x = np.ldexp(np.ones(k.size), k).astype(np.float32)
    assert _ulps(cf.p_log(x), k * np.log(2.0)).max() <= 1.0


def test_p_rsq_within_1p5_ulp():
    g = np.random.default_rng(13)
    x = np.exp(g.uniform(-80, 80, 300_000)).astype(np.float32)
    e = _ulps(cf.p_rsq(x), 1.0 / np.sqrt(x.astype(np.float64)))
    assert e.max() <= 1.5
    assert cf.p_rsq(np.float32(4.0)) == np.float32(0.5)


def test_pairwise_tree_order_decides():
    # sequential: ((((1e8 + 1) - 1e8) + 1) + 1) = 2; the fixed tree ((a0+a1)+(a2+a3))+a4 gives 1
    v = [np.float32(x) for x in (1e8, 1.0, -1e8, 1.0, 1.0)]
    assert cf._pairwise_in_place(v) == np.float32(1.0)
    assert cf._pairwise_in_place(v[:1]) == v[0]


def _dyadic(T, H, V, cfg):
    h = datagen.dyadic_bf16(T, H, cfg, datagen.TID_HIDDEN, k_max=4, log2_den=2)
    W = datagen.dyadic_bf16(V, H, cfg, datagen.TID_W, k_max=4, log2_den=4)
    y = datagen.uniform_targets(T, V, cfg)
    return h, W, y


@pytest.mark.parametrize("T,H,V,S,tau,ent", [
    (37, 256, 3000, 4, 0.7, True),    # 4 segments of 750 = 11 tiles + 46
    (20, 128, 9000, 1, 1.0, True),    # 141 tiles: 5 fold groups, tree with pass-through
    (9, 384, 5600, 8, 1.0, False),    # 8 segments of 700
])
def test_model_matches_oracle(T, H, V, S, tau, ent):
    h, W, y = _dyadic(T, H, V, 300 + S)
    y[::5] = -1
    z = cf.exact_logits(h, W)
    got = cf.forward(z, y, S, inv_tau=float(np.float32(1.0 / tau)), entropy=ent)
    want = oracle.logprob(h, W, y, tau=tau, want_entropy=ent)
    for k in (("logp", "lse", "entropy") if ent else ("logp", "lse")):
        d = np.abs(got[k].astype(np.float64) - want[k])
        assert d.max() <= 2e-5, (k, d.max())
    assert np.all(got["logp"][y < 0] == 0.0) and not np.any(np.signbit(got["lse"][y < 0]))


def test_model_rmsnorm_matches_oracle():
    T, H = 24, 512
    x = datagen.dyadic_bf16(T, H, 310, datagen.TID_HIDDEN, k_max=4, log2_den=0)
    gk = datagen.dyadic_bf16(1, H, 310, datagen.TID_GAMMA, k_max=4, log2_den=3)[0]
    g = datagen.f32_to_bf16_bits(cf.bf16_to_f32(gk) + np.float32(1.0))
    got = cf.bf16_to_f32(cf.rmsnorm_bits(x, g, 1e-6)).astype(np.float64)
    want = oracle.rmsnorm_bf16(oracle.bf16_bits_to_f64(x), oracle.bf16_bits_to_f64(g), 1e-6)
    rel = np.abs(got - want) / np.maximum(np.abs(want), 1e-30)
    assert rel.max() <= 2.0 ** -8  # at most one bf16 rounding step apart
    assert np.mean(got != want) < 0.02


def test_exact_logits_refuses_inexact_inputs():
    h, W, _ = datagen.small_case(4, 256, 100, 320)
    with pytest.raises(AssertionError):
        cf.exact_logits(h, W)
