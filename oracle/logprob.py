"""Float64 oracle of the selected-token logprob (test infrastructure; see package docstring).

Notation: h[t,k] hidden row, W[v,k] LM-head row, z[t,v] = sum_k h[t,k] W[v,k] the logit,
z' = z / tau the tempered logit (tau = 1 unless a workload says otherwise), y_t the target token.

    lse_t   = M_t + log sum_v exp(z'_tv - M_t),     M_t = max_v z'_tv
    logp_t  = z'_{t,y_t} - lse_t
    ent_t   = lse_t - sum_v exp(z'_tv - lse_t) z'_tv          (Shannon entropy, nats)
    y_t < 0 (a padded row): logp_t = lse_t = ent_t = 0

Sources: log_softmax then the target's value, with its max and sum reductions (nxbn.cn blog,
§3.1); "Linear logprob" row of the strict-path boundary table and the "logprobs" item of the ROCm
fixes list (RL-Kernel v0.1.0 summary page); recomputing the logprob of the rollout's token from the
same weights (aihirek.info report, "Miért térhet el ugyanaz a modell?"). Entropy and temperature
are not on the pages; they are the norm_head workload's extra outputs (tempered softmax entropy).
The final RMSNorm is the "RMSNorm" row of the same boundary table (reduction domain, epsilon,
output boundary); its bf16 output is the one dtype boundary this oracle models, because it defines
the LM head's input.
"""

from __future__ import annotations

from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np

# Which functions are pinned by what (tests/test_oracle.py holds each pin).
PINS = {
    "bf16_bits_to_f64": "known bit patterns; torch bfloat16->float64 conversion",
    "round_to_bf16": "hand-worked ties/halfway cases; torch float32->bfloat16 RNE on fp32 inputs",
    "rmsnorm_bf16": "constant rows (x/|x| closed form), eps=0 textbook x/rms(x), a 3-4 row",
    "logits": "exact rational dot products (Fraction) on small integer bf16 inputs",
    "logsumexp_rows": "uniform logits give log V; shift invariance; Decimal brute force",
    "log_softmax_rows": "sum_v exp(logp_v) = 1 within 1e-12; V=2 closed form; geometric series",
    "select_logprob": "V=2 closed form; arithmetic-progression closed form per target; masks",
    "entropy_rows": "uniform gives log V; binary entropy closed form; one large logit",
    "logprob": "all of the above composed; Decimal brute force on tiny exact inputs",
    "sample_targets": "inverse CDF on a hand-worked 3-token distribution",
}


# ------------------------------------------------------------------------------------------
# bfloat16 <-> float64
# ------------------------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of each bfloat16 bit pattern, as float64.

    A bfloat16 is the top 16 bits of an IEEE binary32, so the value is that of the binary32 with
    the low 16 bits zero; binary32 -> binary64 is exact.
    """
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value of each float64, ties to even (one rounding, straight from fp64).

    bfloat16 keeps 8 significant bits. With x = m * 2**e and 0.5 <= |m| < 1 the representable
    neighbours are multiples of 2**(e-8); below the smallest normal (2**-126) the spacing stays
    2**-133. Finite inputs only.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    scaled = np.ldexp(x, 8 - e)
    return np.ldexp(np.rint(scaled), e - 8)


# ------------------------------------------------------------------------------------------
# RMSNorm (norm_head workload)
# ------------------------------------------------------------------------------------------

def rmsnorm_bf16(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """y = bf16( x * gamma / sqrt(mean_k x_k**2 + eps) ), exact fp64 up to the one bf16 rounding.

    x: float64 [T, H]; gamma: float64 [H]. No residual add (the workload has none).
    """
    ms = np.mean(x * x, axis=1, keepdims=True)
    return round_to_bf16(x * gamma[None, :] / np.sqrt(ms + eps))


# ------------------------------------------------------------------------------------------
# Logits and the per-row reductions
# ------------------------------------------------------------------------------------------

def logits(h: np.ndarray, W: np.ndarray) -> np.ndarray:
    """z = h W^T in float64 (h [T,H], W [V,H]); one library matmul."""
    return np.asarray(h, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def logsumexp_rows(zp: np.ndarray) -> np.ndarray:
    """lse_t = M_t + log sum_v exp(z'_tv - M_t) over each row of z' (float64)."""
    M = np.max(zp, axis=1)
    return M + np.log(np.sum(np.exp(zp - M[:, None]), axis=1))


def log_softmax_rows(zp: np.ndarray) -> np.ndarray:
    """Full log-softmax z'_tv - lse_t (used by the normalisation and shift pins)."""
    return zp - logsumexp_rows(zp)[:, None]


def entropy_rows(zp: np.ndarray, lse: np.ndarray) -> np.ndarray:
    """H_t = lse_t - sum_v p_tv z'_tv with p_tv = exp(z'_tv - lse_t), in nats."""
    p = np.exp(zp - lse[:, None])
    return lse - np.sum(p * zp, axis=1)


def select_logprob(zp: np.ndarray, targets: np.ndarray, want_entropy: bool = False):
    """(logp, lse, entropy-or-None) of each row of tempered logits z' at its target.

    Rows with a negative target are padding: all their outputs are 0. A target >= V is invalid
    for the oracle and raises.
    """
    zp = np.asarray(zp, dtype=np.float64)
    y = np.asarray(targets, dtype=np.int64)
    T, V = zp.shape
    if np.any(y >= V):
        raise ValueError("target out of range")
    active = y >= 0
    logp = np.zeros(T)
    lse = np.zeros(T)
    ent = np.zeros(T) if want_entropy else None
    if np.any(active):
        za = zp[active]
        l = logsumexp_rows(za)
        lse[active] = l
        logp[active] = za[np.arange(za.shape[0]), y[active]] - l
        if want_entropy:
            ent[active] = entropy_rows(za, l)
    return logp, lse, ent


def logprob(hidden_bits: np.ndarray, W: np.ndarray, targets: np.ndarray, tau: float = 1.0,
            gamma_bits: np.ndarray | None = None, rms_eps: float = 1e-6,
            want_entropy: bool = False, rows: np.ndarray | None = None,
            row_chunk: int = 512) -> dict:
    """The oracle: selected-token logprob (and lse, entropy) of every row, in float64.

    hidden_bits: uint16 bf16 bits [T, H] (or float64 hidden values).
    W: float64 [V, H] (decode once with ``bf16_bits_to_f64``), or uint16 bf16 bits.
    targets: int [T]; negative = padded row.
    gamma_bits: bf16 bits [H] -> apply the final RMSNorm (bf16 output) before the head.
    rows: optional subset of row indices to evaluate (outputs are for those rows only).
    Rows are processed in chunks of ``row_chunk`` only to bound memory; rows are independent.
    """
    Wf = bf16_bits_to_f64(W) if W.dtype == np.uint16 else np.asarray(W, dtype=np.float64)
    hb = np.asarray(hidden_bits)
    y = np.asarray(targets, dtype=np.int64)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        hb = hb[rows]
        y = y[rows]
    gamma = None if gamma_bits is None else bf16_bits_to_f64(gamma_bits)
    T = hb.shape[0]
    out_logp = np.zeros(T)
    out_lse = np.zeros(T)
    out_ent = np.zeros(T) if want_entropy else None
    for r0 in range(0, T, row_chunk):
        r1 = min(T, r0 + row_chunk)
        yc = y[r0:r1]
        act = np.nonzero(yc >= 0)[0]
        if act.size == 0:
            continue
        hc = hb[r0:r1][act]
        h = bf16_bits_to_f64(hc) if hc.dtype == np.uint16 else np.asarray(hc, dtype=np.float64)
        if gamma is not None:
            h = rmsnorm_bf16(h, gamma, rms_eps)
        zp = logits(h, Wf) / tau
        lp, ls, en = select_logprob(zp, yc[act], want_entropy)
        out_logp[r0 + act] = lp
        out_lse[r0 + act] = ls
        if want_entropy:
            out_ent[r0 + act] = en
    res = {"logp": out_logp, "lse": out_lse}
    if want_entropy:
        res["entropy"] = out_ent
    return res


def sample_targets(zp: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Draw one token per row from softmax(z') by inverse CDF with the given uniforms u in [0,1).

    The token is the first v whose cumulative probability exceeds u_t.
    """
    zp = np.asarray(zp, dtype=np.float64)
    p = np.exp(zp - logsumexp_rows(zp)[:, None])
    c = np.cumsum(p, axis=1)
    c[:, -1] = np.inf  # rounding in the cumulative sum must never push u past the last token
    return np.array([int(np.searchsorted(c[i], u[i], side="right")) for i in range(zp.shape[0])],
                    dtype=np.int32)


# ------------------------------------------------------------------------------------------
# Brute force for tiny shapes: exact rational logits, then 60-digit decimal exp/log with no
# max-shift. Structurally independent of the float64 path above.
# ------------------------------------------------------------------------------------------

def logprob_bruteforce(h_vals, W_vals, targets, tau: float = 1.0, want_entropy: bool = False):
    """Pure-Python loops: z as exact Fractions, then log(exp(z'_y) / sum_v exp(z'_v)) in Decimal.

    h_vals [T][H], W_vals [V][H]: Python floats that are exactly bf16 values. Returns float lists.
    """
    T = len(h_vals)
    V = len(W_vals)
    tau_q = Fraction(tau)
    logp, lse, ent = [], [], []
    with localcontext() as ctx:
        ctx.prec = 60
        for t in range(T):
            y = int(targets[t])
            if y < 0:
                logp.append(0.0)
                lse.append(0.0)
                ent.append(0.0)
                continue
            zq = []
            for v in range(V):
                acc = Fraction(0)
                for k in range(len(h_vals[t])):
                    acc += Fraction(h_vals[t][k]) * Fraction(W_vals[v][k])
                zq.append(acc / tau_q)
            zd = [Decimal(q.numerator) / Decimal(q.denominator) for q in zq]
            ex = [d.exp() for d in zd]
            S = sum(ex, Decimal(0))
            l = S.ln()
            logp.append(float((ex[y] / S).ln()))
            lse.append(float(l))
            if want_entropy:
                ent.append(float(-sum(((e / S) * (e / S).ln() for e in ex), Decimal(0))))
            else:
                ent.append(0.0)
    return {"logp": logp, "lse": lse, "entropy": ent}

