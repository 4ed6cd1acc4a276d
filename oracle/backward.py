"""Float64 oracle of the backward of the selected-token logprob (test infrastructure; see the
package docstring).

The training side differentiates the recomputed logprob, so the kernel library that fixes the
forward has to provide its backward too, with numerics just as fixed (nxbn.cn blog, §3.3, on the
training-side integration, and §4.2, whose autograd wrapper routes log_softmax's backward to the
same library). The loss seen by this path is

    L = sum_t g_t logp_t  +  sum_t gH_t ent_t          (g, gH: upstream gradients per row)

and its gradient with respect to the tempered logit z'_tv, with p_tv = exp(z'_tv - lse_t):

    dL/dz'_tv = g_t (delta(v = y_t) - p_tv)  -  gH_t p_tv (z'_tv - lse_t + ent_t)

(d lse/d z'_v = p_v; d ent/d z'_v = -p_v (z'_v - E[z']), E[z'] = lse - ent). Through z' = z / tau:
dz = dz' / tau. Through z = h W^T: dh = dz W and dW = dz^T h. Padded rows (y_t < 0) contribute
nothing.

Rounding point: the library hands dz to its two bf16 GEMMs, so dz is materialized in bf16 (round to
nearest even). ``round_dz=True`` (the default) models that one dtype boundary, exactly as the
forward oracle models the RMSNorm output's bf16 boundary; everything else is exact float64.
``round_dz=False`` gives the exact gradient (what the finite-difference and autograd pins check).
"""

from __future__ import annotations

import numpy as np

from .logprob import bf16_bits_to_f64, entropy_rows, logsumexp_rows, rmsnorm_bf16, round_to_bf16

PINS_RMS = {
    "rmsnorm_backward": "torch CPU float64 autograd through x gamma / sqrt(mean x^2 + eps); central "
                        "finite differences; a row x = c (constant) closed form",
}

PINS = {
    "dlogits": "central finite differences of the forward oracle; torch CPU float64 autograd of "
               "log_softmax + gather + entropy; uniform-logit closed form; rows sum to zero",
    "grads (dh, dW)": "central finite differences; torch CPU float64 autograd through h W^T / tau; "
                      "uniform-logit closed form dh = g (W[y] - mean_v W[v]) / tau; sum_v dW[v] = 0",
}


def _f64(x: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f64(x) if x.dtype == np.uint16 else np.asarray(x, dtype=np.float64)


def dlogits(zp: np.ndarray, targets: np.ndarray, g: np.ndarray, gH: np.ndarray | None = None,
            tau: float = 1.0) -> np.ndarray:
    """dL/dz [T, V] from tempered logits z' (float64), without any rounding."""
    zp = np.asarray(zp, dtype=np.float64)
    y = np.asarray(targets, dtype=np.int64)
    T, V = zp.shape
    if np.any(y >= V):
        raise ValueError("target out of range")
    out = np.zeros((T, V))
    act = np.nonzero(y >= 0)[0]
    if act.size == 0:
        return out
    za = zp[act]
    lse = logsumexp_rows(za)
    p = np.exp(za - lse[:, None])
    d = -p
    d[np.arange(act.size), y[act]] += 1.0
    d *= np.asarray(g, dtype=np.float64)[act, None]
    if gH is not None:
        ent = entropy_rows(za, lse)
        d -= np.asarray(gH, dtype=np.float64)[act, None] * p * (za - lse[:, None] + ent[:, None])
    out[act] = d / tau
    return out


def rmsnorm_backward(x: np.ndarray, gamma: np.ndarray, eps: float, dy: np.ndarray):
    """(dx, dgamma) of y = x gamma / sqrt(mean_k x_k^2 + eps), given dy (float64, per row).

    With r = (mean x^2 + eps)^(-1/2) and c = sum_j dy_j gamma_j x_j:
        dx_k = r gamma_k dy_k - x_k r^3 c / H,      dgamma_k = sum_t dy_tk x_tk r_t.
    The bf16 rounding of y in the forward is passed straight through (its derivative is taken
    as 1), as the library does.
    """
    x = np.asarray(x, dtype=np.float64)
    H = x.shape[1]
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps)
    c = np.sum(dy * gamma[None, :] * x, axis=1)
    dx = (r[:, None] * gamma[None, :] * dy) - x * (r ** 3 * c / H)[:, None]
    dgamma = np.sum(dy * x * r[:, None], axis=0)
    return dx, dgamma


def grads(hidden: np.ndarray, W: np.ndarray, targets: np.ndarray, grad_logp: np.ndarray,
          grad_entropy: np.ndarray | None = None, tau: float = 1.0, round_dz: bool = True,
          dh_rows: np.ndarray | None = None, dW_rows: np.ndarray | None = None,
          row_chunk: int = 256, gamma_bits: np.ndarray | None = None, rms_eps: float = 1e-6,
          round_y: bool = True) -> dict:
    """dh [T, H] and dW [V, H] of L (and dgamma [H] with the RMSNorm), in float64.

    hidden: bf16 bits [T, H] or float64 values; W: bf16 bits [V, H] or float64 values.
    gamma_bits: apply the final RMSNorm first (as the forward oracle does, its output rounded to
    bf16 unless ``round_y`` is False); dh is then the gradient with respect to the RMSNorm's
    input x, and dW is taken against the normed rows.
    dh_rows / dW_rows: evaluate only those rows of dh / of dW (all rows still enter every lse
    and every dW sum). Rows are processed in chunks of ``row_chunk`` to bound memory.
    """
    x = _f64(hidden)
    gamma = None if gamma_bits is None else _f64(gamma_bits)
    if gamma is None:
        h = x
    elif round_y:
        h = rmsnorm_bf16(x, gamma, rms_eps)
    else:
        h = x * gamma[None, :] / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + rms_eps)
    Wf = _f64(W)
    y = np.asarray(targets, dtype=np.int64)
    g = np.asarray(grad_logp, dtype=np.float64)
    gH = None if grad_entropy is None else np.asarray(grad_entropy, dtype=np.float64)
    T, H = h.shape
    V = Wf.shape[0]
    rows_h = np.arange(T) if dh_rows is None else np.asarray(dh_rows, dtype=np.int64)
    if gamma is not None and dh_rows is not None:
        rows_h = np.arange(T)  # dgamma sums over every row
    rows_w = np.arange(V) if dW_rows is None else np.asarray(dW_rows, dtype=np.int64)
    dh = np.zeros((rows_h.size, H))
    dW = np.zeros((rows_w.size, H))
    want_h = np.zeros(T, dtype=bool)
    want_h[rows_h] = True
    pos_h = np.full(T, -1)
    pos_h[rows_h] = np.arange(rows_h.size)
    for r0 in range(0, T, row_chunk):
        r1 = min(T, r0 + row_chunk)
        zp = (h[r0:r1] @ Wf.T) / tau
        dz = dlogits(zp, y[r0:r1], g[r0:r1], None if gH is None else gH[r0:r1], tau)
        if round_dz:
            dz = round_to_bf16(dz)
        sel = np.nonzero(want_h[r0:r1])[0]
        if sel.size:
            dh[pos_h[r0 + sel]] = dz[sel] @ Wf
        dW += dz[:, rows_w].T @ h[r0:r1]
    if gamma is None:
        return {"dh": dh, "dW": dW}
    dx, dgamma = rmsnorm_backward(x, gamma, rms_eps, dh)
    if dh_rows is not None:
        dx = dx[np.asarray(dh_rows, dtype=np.int64)]
    return {"dh": dx, "dW": dW, "dgamma": dgamma}
