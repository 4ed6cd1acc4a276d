"""Pins of the float64 backward oracle (oracle/backward.py): central finite differences of the
forward oracle, torch CPU float64 autograd (an independent implementation of log_softmax's
backward), the uniform-logit closed form, the zero-sum invariant, padded rows and the bound on the
one modelled rounding point (bf16 dz)."""

import numpy as np
import pytest

import oracle


def _case(T, H, V, seed, pad=()):
    g = np.random.default_rng(seed)
    h = g.normal(size=(T, H))
    W = g.normal(size=(V, H)) * 0.5
    y = g.integers(0, V, size=T)
    y[list(pad)] = -1
    gl = g.normal(size=T)
    ge = g.normal(size=T)
    return h, W, y, gl, ge


def _loss(h, W, y, gl, ge, tau):
    out = oracle.logprob(h, W, y, tau=tau, want_entropy=True)
    return float(np.dot(gl, out["logp"]) + np.dot(ge, out["entropy"]))


@pytest.mark.parametrize("tau,use_ent", [(1.0, False), (0.7, True)])
def test_grads_match_central_differences(tau, use_ent):
    T, H, V = 3, 6, 11
    h, W, y, gl, ge = _case(T, H, V, 1, pad=(1,))
    ge = ge if use_ent else np.zeros(T)
    got = oracle.grads(h, W, y, gl, ge if use_ent else None, tau=tau, round_dz=False)
    eps = 1e-6
    for arr, key in ((h, "dh"), (W, "dW")):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            lp = _loss(h, W, y, gl, ge, tau)
            arr[idx] = old - eps
            lm = _loss(h, W, y, gl, ge, tau)
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(got[key], num, rtol=1e-6, atol=1e-8)


def test_grads_match_torch_autograd():
    torch = pytest.importorskip("torch")
    T, H, V, tau = 7, 16, 40, 0.8
    h, W, y, gl, ge = _case(T, H, V, 2, pad=(0, 4))
    ht = torch.tensor(h, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    lsm = torch.log_softmax((ht @ Wt.T) / tau, dim=1)
    act = torch.tensor(y >= 0)
    yy = torch.tensor(np.where(y >= 0, y, 0))
    logp = lsm[torch.arange(T), yy]
    ent = -(lsm.exp() * lsm).sum(dim=1)
    L = (torch.tensor(gl) * logp * act).sum() + (torch.tensor(ge) * ent * act).sum()
    L.backward()
    got = oracle.grads(h, W, y, gl, ge, tau=tau, round_dz=False)
    np.testing.assert_allclose(got["dh"], ht.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(got["dW"], Wt.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_uniform_logits_closed_form():
    # h = 0: every logit is 0, p = 1/V, the entropy term (z' - lse + ent) vanishes, and
    # dh_t = g_t (W[y_t] - mean_v W[v]) / tau, dW = 0.
    T, H, V, tau = 4, 8, 13, 0.5
    _, W, y, gl, ge = _case(T, H, V, 3, pad=(2,))
    h = np.zeros((T, H))
    got = oracle.grads(h, W, y, gl, ge, tau=tau, round_dz=False)
    want = np.zeros((T, H))
    for t in range(T):
        if y[t] >= 0:
            want[t] = gl[t] * (W[y[t]] - W.mean(axis=0)) / tau
    np.testing.assert_allclose(got["dh"], want, rtol=1e-13, atol=1e-15)
    assert np.all(got["dW"] == 0.0)


def test_dlogits_rows_sum_to_zero_and_dW_columns_too():
    T, H, V = 6, 10, 50
    h, W, y, gl, ge = _case(T, H, V, 4, pad=(3,))
    zp = h @ W.T / 0.9
    d = oracle.dlogits(zp, y, gl, ge, tau=0.9)
    assert np.abs(d.sum(axis=1)).max() < 1e-13
    assert np.all(d[3] == 0.0)
    got = oracle.grads(h, W, y, gl, ge, tau=0.9, round_dz=False)
    assert np.abs(got["dW"].sum(axis=0)).max() < 1e-12
    assert np.all(got["dh"][3] == 0.0)


def test_padded_rows_do_not_reach_dW():
    T, H, V = 5, 8, 30
    h, W, y, gl, ge = _case(T, H, V, 5, pad=(1, 2))
    a = oracle.grads(h, W, y, gl, ge)
    h2 = h.copy()
    h2[[1, 2]] = 1e3
    b = oracle.grads(h2, W, y, gl, ge)
    assert np.array_equal(a["dW"], b["dW"])


def test_rounded_dz_stays_within_the_bf16_bound():
    T, H, V = 8, 16, 64
    h, W, y, gl, ge = _case(T, H, V, 6)
    ex = oracle.grads(h, W, y, gl, ge, round_dz=False)
    rd = oracle.grads(h, W, y, gl, ge, round_dz=True)
    dz = np.abs(oracle.dlogits(h @ W.T, y, gl, ge))
    bound_h = 2.0 ** -8 * (dz @ np.abs(W))      # half a bf16 ulp of each dz, summed
    bound_w = 2.0 ** -8 * (dz.T @ np.abs(h))
    assert np.all(np.abs(rd["dh"] - ex["dh"]) <= bound_h + 1e-300)
    assert np.all(np.abs(rd["dW"] - ex["dW"]) <= bound_w + 1e-300)
    assert not np.array_equal(rd["dh"], ex["dh"])


def test_row_subsets_equal_the_full_result():
    T, H, V = 9, 8, 40
    h, W, y, gl, ge = _case(T, H, V, 7)
    full = oracle.grads(h, W, y, gl, ge, row_chunk=4)
    sub = oracle.grads(h, W, y, gl, ge, dh_rows=np.array([0, 5, 8]), dW_rows=np.array([3, 39]))
    np.testing.assert_allclose(sub["dh"], full["dh"][[0, 5, 8]], rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(sub["dW"], full["dW"][[3, 39]], rtol=1e-14, atol=1e-16)


def _rms_case(T, H, V, seed):
    g = np.random.default_rng(seed)
    x = g.normal(size=(T, H))
    gamma = 1.0 + 0.1 * g.normal(size=H)
    W = g.normal(size=(V, H)) * 0.3
    y = g.integers(0, V, size=T)
    return x, gamma, W, y, g.normal(size=T), g.normal(size=T)


def test_rmsnorm_grads_match_torch_autograd():
    torch = pytest.importorskip("torch")
    T, H, V, tau, eps = 6, 16, 30, 0.7, 1e-3
    x, gamma, W, y, gl, ge = _rms_case(T, H, V, 11)
    y[2] = -1
    xt = torch.tensor(x, requires_grad=True)
    gt = torch.tensor(gamma, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    hn = xt * gt / torch.sqrt((xt * xt).mean(dim=1, keepdim=True) + eps)
    lsm = torch.log_softmax((hn @ Wt.T) / tau, dim=1)
    act = torch.tensor(y >= 0)
    yy = torch.tensor(np.where(y >= 0, y, 0))
    L = (torch.tensor(gl) * lsm[torch.arange(T), yy] * act).sum() \
        + (torch.tensor(ge) * -(lsm.exp() * lsm).sum(dim=1) * act).sum()
    L.backward()
    got = oracle.grads(x, W, y, gl, ge, tau=tau, round_dz=False, gamma_bits=gamma, rms_eps=eps,
                       round_y=False)
    np.testing.assert_allclose(got["dh"], xt.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(got["dW"], Wt.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(got["dgamma"], gt.grad.numpy(), rtol=1e-11, atol=1e-13)


def test_rmsnorm_backward_central_differences():
    T, H, eps = 3, 5, 1e-2
    g = np.random.default_rng(12)
    x = g.normal(size=(T, H))
    gamma = 1.0 + 0.2 * g.normal(size=H)
    dy = g.normal(size=(T, H))

    def f(xx, gg):
        yv = xx * gg[None, :] / np.sqrt(np.mean(xx * xx, axis=1, keepdims=True) + eps)
        return float(np.sum(dy * yv))

    dx, dgam = oracle.rmsnorm_backward(x, gamma, eps, dy)
    e = 1e-6
    for arr, want in ((x, dx), (gamma, dgam)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + e
            fp = f(x, gamma)
            arr[idx] = old - e
            fm = f(x, gamma)
            arr[idx] = old
            num[idx] = (fp - fm) / (2 * e)
        np.testing.assert_allclose(want, num, rtol=1e-6, atol=1e-9)


def test_rmsnorm_backward_constant_row():
    # a constant row x = c 1 with eps = 0 gives y = gamma sign(c): r = 1/|c|, so with dy = 1,
    # dx_k = gamma_k / |c| - c r^3 (c sum gamma) / H and dgamma_k = sign(c); y does not change
    # when x is scaled, so dx is orthogonal to x.
    H = 6
    gamma = np.linspace(0.5, 1.5, H)
    x = np.full((1, H), -3.0)
    dy = np.ones((1, H))
    dx, dgam = oracle.rmsnorm_backward(x, gamma, 0.0, dy)
    # r = 1/3; c = -3 sum(gamma); dx_k = gamma_k/3 - (-3)(1/27)(-3 sum gamma)/H
    want = gamma / 3 - np.sum(gamma) / (3 * H)
    np.testing.assert_allclose(dx[0], want, rtol=1e-14)
    np.testing.assert_allclose(dgam, -np.ones(H), rtol=1e-14)
    assert abs(np.dot(dx[0], np.ones(H))) < 1e-13  # scaling x leaves y unchanged
