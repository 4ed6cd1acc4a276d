"""Pins of the CPU oracle against facts the mathematics fixes (no GPU).

Each test checks the oracle against something other than itself: hand-worked values, closed forms,
a library conversion, or an exact rational / 60-digit decimal brute force.
"""

import math

import numpy as np
import pytest
import torch

import oracle


# ------------------------------------------------------------------ bfloat16 decode / encode

def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xBF80, 0x4000, 0x3F81, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x3E80],
                    dtype=np.uint16)
    want = [1.0, -1.0, 2.0, 1.0 + 2.0 ** -7, 0.0, -0.0, (2.0 - 2.0 ** -7) * 2.0 ** 127,
            2.0 ** -133, 0.25]
    got = oracle.bf16_bits_to_f64(bits)
    assert list(got) == want


def test_bf16_decode_matches_torch():
    g = np.random.default_rng(7)
    bits = g.integers(0, 1 << 16, size=20000).astype(np.uint16)
    exp_field = (bits >> 7) & 0xFF
    bits = bits[exp_field != 0xFF]  # finite only
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), ref.numpy())


def test_round_to_bf16_hand_cases():
    cases = {
        1.0 + 2.0 ** -8: 1.0,                          # halfway, 1.0 is even
        1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,           # halfway, up to the even neighbour
        1.0 + 2.0 ** -8 + 2.0 ** -30: 1.0 + 2.0 ** -7,  # just above halfway
        -(1.0 + 2.0 ** -8): -1.0,
        0.84853: 434 * 2.0 ** -9,
        3.0 * 2.0 ** -130: 3.0 * 2.0 ** -130,            # bf16 subnormal, exact
        0.0: 0.0,
        255.5: 256.0,                                   # carries into the next binade
    }
    for x, want in cases.items():
        assert oracle.round_to_bf16(np.array([x]))[0] == want, x


def test_round_to_bf16_matches_torch_rne_on_fp32():
    g = np.random.default_rng(11)
    x32 = (g.standard_normal(50000) * np.exp(g.uniform(-20, 20, 50000))).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_to_bf16(x32.astype(np.float64)), ref)


# ------------------------------------------------------------------ RMSNorm

def test_rmsnorm_three_four_row():
    # rms([3,4]) = sqrt(12.5); 3/3.5355 = 0.848528 -> 434 * 2^-9; 4/3.5355 = 1.131371 -> 145 * 2^-7
    y = oracle.rmsnorm_bf16(np.array([[3.0, 4.0]]), np.array([1.0, 1.0]), 0.0)
    assert list(y[0]) == [434 * 2.0 ** -9, 145 * 2.0 ** -7]
    # gamma multiplies before the single rounding: 2 * 0.848528 -> 217 * 2^-7
    y2 = oracle.rmsnorm_bf16(np.array([[3.0, 4.0]]), np.array([2.0, 1.0]), 0.0)
    assert y2[0, 0] == 217 * 2.0 ** -7


def test_rmsnorm_constant_rows_and_eps_inside_sqrt():
    H = 64
    x = np.full((3, H), 0.0)
    x[0] = 2.5
    x[1] = -7.0
    x[2] = 1e-3
    y = oracle.rmsnorm_bf16(x, np.ones(H), 0.0)
    assert np.all(y[0] == 1.0) and np.all(y[1] == -1.0) and np.all(y[2] == 1.0)
    # eps = c^2: c / sqrt(c^2 + eps) = 1/sqrt(2) = 0.7071068 -> 362 * 2^-9
    ye = oracle.rmsnorm_bf16(x[2:3], np.ones(H), 1e-6)
    assert np.all(ye == 362 * 2.0 ** -9)


# ------------------------------------------------------------------ logits

def test_logits_exact_integer_dot_products():
    g = np.random.default_rng(3)
    h = g.integers(-8, 9, size=(5, 7)).astype(np.float64)
    W = g.integers(-8, 9, size=(11, 7)).astype(np.float64)
    z = oracle.logits(h, W)
    assert z.shape == (5, 11)
    for t in range(5):
        for v in range(11):
            assert z[t, v] == sum(int(h[t, k]) * int(W[v, k]) for k in range(7))


# ------------------------------------------------------------------ reductions

@pytest.mark.parametrize("V", [1000, 151936])
def test_uniform_logits_give_minus_log_V(V):
    z = np.zeros((3, V))
    y = np.array([0, V // 2, V - 1])
    logp, lse, ent = oracle.select_logprob(z, y, want_entropy=True)
    assert np.allclose(logp, -math.log(V), rtol=0, atol=1e-12)
    assert np.allclose(lse, math.log(V), rtol=0, atol=1e-12)
    assert np.allclose(ent, math.log(V), rtol=0, atol=1e-10)
    c = np.full((1, V), 3.7)
    assert abs(oracle.logsumexp_rows(c)[0] - (3.7 + math.log(V))) < 1e-12


def test_uniform_closed_form_values():
    assert abs(-math.log(1000) - (-6.907755278982137)) < 1e-15
    assert abs(-math.log(151936) - (-11.931214658529285)) < 1e-14
    logp, _, _ = oracle.select_logprob(np.zeros((1, 1000)), np.array([5]))
    assert abs(logp[0] - (-6.907755278982137)) < 1e-13


def test_normalisation_and_shift_invariance():
    g = np.random.default_rng(5)
    z = g.standard_normal((4, 5000)) * 3.0
    lsm = oracle.log_softmax_rows(z)
    assert np.all(np.abs(np.exp(lsm).sum(axis=1) - 1.0) < 1e-12)
    for c in (-50.0, 1e-3, 123.0):
        lsm2 = oracle.log_softmax_rows(z + c)
        assert np.max(np.abs(lsm2 - lsm) / np.maximum(1.0, np.abs(lsm))) < 1e-12


def test_two_token_closed_form():
    z = np.array([[0.3, -1.2], [5.0, 5.5], [-20.0, 3.0]])
    for y in (0, 1):
        logp, _, _ = oracle.select_logprob(z, np.array([y, y, y]))
        other = 1 - y
        want = -np.log1p(np.exp(z[:, other] - z[:, y]))
        assert np.allclose(logp, want, rtol=0, atol=1e-14)


def test_arithmetic_progression_closed_form_pins_the_gather_index():
    V = 777
    a = 0.013
    z = (a * np.arange(V))[None, :].repeat(5, axis=0)
    y = np.array([0, 1, 100, 500, V - 1])
    lse_closed = math.log((math.exp(a * V) - 1.0) / (math.exp(a) - 1.0))
    logp, lse, _ = oracle.select_logprob(z, y)
    assert np.allclose(lse, lse_closed, rtol=0, atol=1e-12)
    assert np.allclose(logp, a * y - lse_closed, rtol=0, atol=1e-12)


def test_entropy_closed_forms():
    # binary entropy of p = sigmoid(d)
    d = 0.8
    p = 1.0 / (1.0 + math.exp(-d))
    want = -(p * math.log(p) + (1 - p) * math.log(1 - p))
    _, _, ent = oracle.select_logprob(np.array([[d, 0.0]]), np.array([0]), want_entropy=True)
    assert abs(ent[0] - want) < 1e-14
    # one logit at +100 among V-1 zeros
    V = 1000
    z = np.zeros((1, V))
    z[0, 17] = 100.0
    r = (V - 1) * math.exp(-100.0)
    lse_c = 100.0 + math.log1p(r)
    ent_c = lse_c - 100.0 / (1.0 + r)
    logp, lse, ent = oracle.select_logprob(z, np.array([17]), want_entropy=True)
    assert abs(lse[0] - lse_c) < 1e-12 and abs(ent[0] - ent_c) < 1e-12
    assert abs(logp[0] - (-math.log1p(r))) < 1e-14
    assert 0.0 <= ent[0] < 1e-38


def test_masked_rows_are_zero():
    z = np.random.default_rng(1).standard_normal((4, 50))
    logp, lse, ent = oracle.select_logprob(z, np.array([3, -1, 7, -5]), want_entropy=True)
    for a in (logp, lse, ent):
        assert a[1] == 0.0 and a[3] == 0.0
        assert a[0] != 0.0 and a[2] != 0.0
    with pytest.raises(ValueError):
        oracle.select_logprob(z, np.array([50, 0, 0, 0]))


def test_invariants_on_random_rows():
    g = np.random.default_rng(9)
    z = g.standard_normal((64, 3000)) * 2.0
    y = g.integers(0, 3000, size=64)
    logp, lse, ent = oracle.select_logprob(z, y, want_entropy=True)
    assert np.all(logp <= 0.0)
    assert np.all(lse >= z.max(axis=1))
    assert np.all(ent >= 0.0) and np.all(ent <= math.log(3000) + 1e-12)


# ------------------------------------------------------------------ end to end vs brute force

def _bits(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_logprob_matches_decimal_bruteforce_on_exact_small_inputs():
    g = np.random.default_rng(21)
    T, H, V = 4, 8, 12
    h = g.integers(-3, 4, size=(T, H)).astype(np.float32) * 0.25
    W = g.integers(-4, 5, size=(V, H)).astype(np.float32) * 0.125
    y = np.array([0, 5, -1, 11])
    for tau in (1.0, 0.7):
        res = oracle.logprob(_bits(h), _bits(W), y, tau=tau, want_entropy=True)
        bf = oracle.logprob_bruteforce(h.tolist(), W.tolist(), y, tau=tau, want_entropy=True)
        for key in ("logp", "lse", "entropy"):
            assert np.allclose(res[key], bf[key], rtol=0, atol=1e-13), (key, tau)


def test_logprob_matches_bruteforce_on_random_bf16():
    T, H, V = 3, 16, 20
    g = np.random.default_rng(33)
    hb = _bits(g.standard_normal((T, H)).astype(np.float32))
    Wb = _bits((g.standard_normal((V, H)) * 0.5).astype(np.float32))
    y = np.array([19, 0, 7])
    hv = oracle.bf16_bits_to_f64(hb).tolist()
    Wv = oracle.bf16_bits_to_f64(Wb).tolist()
    res = oracle.logprob(hb, Wb, y)
    bf = oracle.logprob_bruteforce(hv, Wv, y)
    assert np.allclose(res["logp"], bf["logp"], rtol=0, atol=1e-13)
    assert np.allclose(res["lse"], bf["lse"], rtol=0, atol=1e-13)


def test_temperature_two_token_end_to_end():
    # h = [1], W = [[a], [b]] -> z = (a, b); z' = z / 0.7
    a, b = 1.5, -0.25
    res = oracle.logprob(_bits(np.array([[1.0]], np.float32)),
                         _bits(np.array([[a], [b]], np.float32)), np.array([0]), tau=0.7)
    assert abs(res["logp"][0] - (-math.log1p(math.exp((b - a) / 0.7)))) < 1e-14


def test_rows_subset_and_chunking_do_not_change_rows():
    g = np.random.default_rng(4)
    hb = _bits(g.standard_normal((40, 32)).astype(np.float32))
    Wb = _bits((g.standard_normal((300, 32)) * 0.1).astype(np.float32))
    y = g.integers(-1, 300, size=40)
    full = oracle.logprob(hb, Wb, y, row_chunk=512)
    one = oracle.logprob(hb, Wb, y, row_chunk=1)
    assert np.array_equal(full["logp"], one["logp"])
    rows = np.array([39, 3, 17])
    sub = oracle.logprob(hb, Wb, y, rows=rows)
    assert np.array_equal(sub["logp"], full["logp"][rows])


def test_rmsnorm_path_end_to_end_constant_rows():
    # gamma = 1 and a constant row normalise to +-1 (eps negligible at bf16 precision here), so
    # z = sum_k W[v,k] * sign; compare with the plain head on the +-1 row.
    H, V = 64, 40
    g = np.random.default_rng(8)
    x = np.zeros((2, H), np.float32)
    x[0] = 3.0
    x[1] = -0.5
    Wb = _bits((g.standard_normal((V, H)) * 0.1).astype(np.float32))
    y = np.array([4, 9])
    normed = oracle.logprob(_bits(x), Wb, y, gamma_bits=_bits(np.ones(H, np.float32)),
                            rms_eps=1e-6)
    plain = oracle.logprob(_bits(np.sign(x)), Wb, y)
    assert np.allclose(normed["logp"], plain["logp"], rtol=0, atol=1e-15)


def test_sample_targets_inverse_cdf():
    zp = np.log(np.array([[0.2, 0.5, 0.3]] * 5))
    u = np.array([0.19, 0.21, 0.69, 0.71, 0.999])
    assert list(oracle.sample_targets(zp, u)) == [0, 1, 1, 2, 2]
