"""A float32 CPU model of the library's numeric contract in its portable mode.

Test infrastructure only. It restates, step by step in numpy float32 (every operation an IEEE
binary32 operation rounded to nearest even), the rules the library fixes for one forward: the
tile statistics over 64-column vocab tiles, the segment fold in groups of 32 tiles, the
cross-segment merge, the optional RMSNorm, and the software EXP, LOG and RSQ of the portable mode.
The pages ask for exactly this kind of contract: a forward whose split, merge order, rounding
points and primitives are fixed (RL-Kernel v0.1.0 summary page, "Numeric execution contract";
nxbn.cn blog, sections 3.2 and 4.3 on fixed in-thread sums and fixed trees). It does not compute
the logits' GEMM in float32: it takes the logits from an exact float64 product of inputs chosen
so that every partial sum is exact in fp32 (see ``exact_logits``), where any summation order gives
the same bits. It shares no code with the HIP library and none with the float64 oracle.
"""

from __future__ import annotations

import numpy as np

F = np.float32
I = np.int32
U = np.uint32

LOG2E = F(float.fromhex("0x1.715476p+0"))
LN2_C1 = F(float.fromhex("0x1.63p-1"))       # 0.693359375: 9 significant bits
LN2_C2 = F(float.fromhex("-0x1.bd0106p-13"))  # fl32(ln 2 - C1)
EXP_HI = F(float.fromhex("0x1.62e430p+6"))    # fl32(ln FLT_MAX)
EXP_LO = F(float.fromhex("-0x1.9fe368p+6"))   # fl32(ln 2^-150)
SQRT2 = F(float.fromhex("0x1.6a09e6p+0"))
INV_FACT = [F(float.fromhex(h)) for h in
            ("0x1.a01a02p-13", "0x1.6c16c2p-10", "0x1.111112p-7", "0x1.555556p-5",
             "0x1.555556p-3")]  # 1/7! .. 1/3!
TWO_OVER_ODD = [F(float.fromhex(h)) for h in
                ("0x1.745d18p-3", "0x1.c71c72p-3", "0x1.24924ap-2", "0x1.99999ap-2",
                 "0x1.555556p-1")]  # 2/11 .. 2/3
TILE = 64
FOLD_GROUP = 32


def _f32(x) -> np.ndarray:
    return np.asarray(x, dtype=F)


def _pow2(n: np.ndarray) -> np.ndarray:
    """2^n as float32 from its exponent field, for normal n (-126 <= n <= 127)."""
    return ((np.asarray(n, dtype=I) + I(127)) << I(23)).astype(I).view(F)


def p_exp(x) -> np.ndarray:
    """e^x: Cody-Waite reduction x = n ln2 + r, Taylor polynomial of e^r to r^7/7!, exact
    scaling by 2^n (two steps near overflow and in the subnormal range, each result rounded once).
    """
    x = _f32(x)
    with np.errstate(invalid="ignore", over="ignore"):
        xc = np.fmin(np.fmax(x, EXP_LO), EXP_HI)
        nf = np.rint(xc * LOG2E)
        n = nf.astype(I)
        r = (xc - nf * LN2_C1) - nf * LN2_C2
        p = np.full_like(r, INV_FACT[0])
        for c in INV_FACT[1:] + [F(0.5), F(1.0), F(1.0)]:
            p = p * r + c
        n2 = np.where(n < -126, I(-64), np.where(n > 127, I(1), I(0))).astype(I)
        y = (p * _pow2(n - n2)) * _pow2(n2)
        y = np.where(x < EXP_LO, F(0.0), y)
        y = np.where(x > EXP_HI, F(np.inf), y)
        y = np.where(np.isnan(x), x, y)
    return y.astype(F)


def p_log(x) -> np.ndarray:
    """log x: x = (1 + f) 2^k with 1 + f in [sqrt(1/2), sqrt(2)]; log(1 + f) = 2 atanh(s),
    s = f / (2 + f), arranged as f - (f^2/2 - s (f^2/2 + R)), R = sum over j = 1..5 of
    2 s^(2j) / (2j + 1); then k C1 + (that + k C2)."""
    x = _f32(x)
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        sub = x < F(2.0 ** -126)
        xs = np.where(sub, x * F(2.0 ** 23), x)
        u = np.ascontiguousarray(xs).view(U)
        k = ((u >> U(23)) & U(0xFF)).astype(I) - I(127) + np.where(sub, I(-23), I(0))
        m = ((u & U(0x007FFFFF)) | U(0x3F800000)).view(F)
        big = m > SQRT2
        m = np.where(big, m * F(0.5), m)
        k = k + big.astype(I)
        f = m - F(1.0)
        s = f / (f + F(2.0))
        z = s * s
        R = np.full_like(z, TWO_OVER_ODD[0])
        for c in TWO_OVER_ODD[1:]:
            R = R * z + c
        R = R * z
        hfsq = F(0.5) * (f * f)
        kf = k.astype(F)
        y = kf * LN2_C1 + (f - (hfsq - (s * (hfsq + R) + kf * LN2_C2)))
        y = np.where(x == F(0.0), F(-np.inf), y)
        y = np.where(x == F(np.inf), F(np.inf), y)
        y = np.where(np.isnan(x) | (x < F(0.0)), F(np.nan), y)
    return y.astype(F)


def p_rsq(x) -> np.ndarray:
    """1 / sqrt(x), both correctly rounded."""
    return (F(1.0) / np.sqrt(_f32(x))).astype(F)


# ------------------------------------------------------------------------------------------
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(U) << U(16)).view(F)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=F).view(U)
    nan = (u & U(0x7FFFFFFF)) > U(0x7F800000)
    r = ((u + U(0x7FFF) + ((u >> U(16)) & U(1))) >> U(16)).astype(np.uint16)
    return np.where(nan, ((u >> U(16)) | U(0x40)).astype(np.uint16), r)


def rmsnorm_bits(x_bits: np.ndarray, gamma_bits: np.ndarray, eps: float) -> np.ndarray:
    """The optional final RMSNorm: per row, lane l of 64 sums x^2 over the 8-element groups
    l, l+64, .. in order; a butterfly over lanes at distances 32 .. 1; r = RSQ(ss fl32(1/H) + eps);
    y = bf16((x r) gamma)."""
    x = bf16_to_f32(x_bits)
    g = bf16_to_f32(gamma_bits)
    T, H = x.shape
    groups = x.reshape(T, H // 8, 8)
    lanes = np.zeros((T, 64), dtype=F)
    for p in range(H // 8):
        for e in range(8):
            v = groups[:, p, e]
            lanes[:, p % 64] = lanes[:, p % 64] + v * v
    for d in (32, 16, 8, 4, 2, 1):
        lanes = lanes + lanes[:, np.arange(64) ^ d]
    inv_h = F(1.0) / F(H)
    r = p_rsq(lanes[:, 0] * inv_h + F(eps))
    return f32_to_bf16_rne((x * r[:, None]) * g[None, :])


def _grid(bits: np.ndarray) -> tuple[int, float]:
    """(a, max |x|): the smallest a with every value an integer multiple of 2^-a."""
    present = np.nonzero(np.bincount(np.asarray(bits, dtype=np.uint16).ravel(),
                                     minlength=65536))[0].astype(np.uint16)
    v = bf16_to_f32(present).astype(np.float64)
    assert np.all(np.isfinite(v)), "non-finite input"
    for a in range(0, 160):
        if np.all(np.ldexp(v, a) == np.round(np.ldexp(v, a))):
            return a, float(np.abs(v).max())
    raise AssertionError("input not on a dyadic grid")


def exact_logits(h_bits: np.ndarray, W_bits: np.ndarray, chunk: int = 16384) -> np.ndarray:
    """z = h W^T, asserting first that it is exact in fp32 under any summation order: h lies on
    the grid 2^-a and W on 2^-b, and max_t sum_k |h_tk| max|W| < 2^(24 - a - b), so every partial
    sum of products is an integer multiple of 2^-(a+b) below 2^24 of them."""
    a, _ = _grid(h_bits)
    b, wmax = _grid(W_bits)
    h = bf16_to_f32(h_bits).astype(np.float64)
    bound = float(np.abs(h).sum(axis=1).max()) * wmax if h.size else 0.0
    assert np.ldexp(bound, a + b) < 2.0 ** 24, "inputs do not give exact fp32 logits"
    V = W_bits.shape[0]
    z = np.empty((h.shape[0], V), dtype=F)
    for v0 in range(0, V, chunk):
        zc = h @ bf16_to_f32(W_bits[v0:v0 + chunk]).astype(np.float64).T
        z[:, v0:v0 + chunk] = zc
        assert np.all(z[:, v0:v0 + chunk].astype(np.float64) == zc)
    return z


# ------------------------------------------------------------------------------------------
def _tile_stats(zs: np.ndarray, entropy: bool):
    """Per 64-column tile of one segment [T, L]: m, s, u (the in-tile rules: max; four lane
    groups g summing their 16 columns 16b + 4g + r sequentially over (b, r); (p0 + p1) +
    (p2 + p3))."""
    T, L = zs.shape
    n = (L + TILE - 1) // TILE
    zp = np.zeros((T, n * TILE), dtype=F)
    zp[:, :L] = zs
    valid = np.zeros(n * TILE, dtype=bool)
    valid[:L] = True
    z5 = zp.reshape(T, n, 4, 4, 4)        # [t, tile, b, g, r]: column 16b + 4g + r
    v5 = valid.reshape(n, 4, 4, 4)[None]
    m = np.where(v5, z5, F(-np.inf)).max(axis=(2, 3, 4))
    d = z5 - m[:, :, None, None, None]
    e = np.where(v5, p_exp(d), F(0.0))
    q = np.where(v5, e * d, F(0.0)) if entropy else None
    ps = np.zeros((T, n, 4), dtype=F)
    pq = np.zeros((T, n, 4), dtype=F)
    for b in range(4):
        for r in range(4):
            ps = ps + e[:, :, b, :, r]
            if entropy:
                pq = pq + q[:, :, b, :, r]
    s = (ps[..., 0] + ps[..., 1]) + (ps[..., 2] + ps[..., 3])
    u = (pq[..., 0] + pq[..., 1]) + (pq[..., 2] + pq[..., 3])
    return m, s, u


def _pairwise_in_place(vals: list[np.ndarray]) -> np.ndarray:
    """Balanced pairwise tree in index order, a missing right member passing the left through."""
    vals = list(vals)
    st = 1
    while st < len(vals):
        for i in range(0, len(vals) - st, 2 * st):
            vals[i] = vals[i] + vals[i + st]
        st *= 2
    return vals[0]


def _segment_fold(m, s, u, entropy: bool):
    """M_s = max of the tile maxima; groups of 32 tiles summed sequentially from +0 of
    s_j EXP(m_j - M_s) (and (u_j + s_j (m_j - M_s)) EXP(m_j - M_s)); a pairwise tree over groups."""
    T, n = m.shape
    M = m.max(axis=1)
    A_groups, B_groups = [], []
    for g0 in range(0, n, FOLD_GROUP):
        A = np.zeros(T, dtype=F)
        B = np.zeros(T, dtype=F)
        for j in range(g0, min(n, g0 + FOLD_GROUP)):
            dm = m[:, j] - M
            e = p_exp(dm)
            A = A + s[:, j] * e
            if entropy:
                B = B + (u[:, j] + s[:, j] * dm) * e
        A_groups.append(A)
        B_groups.append(B)
    return M, _pairwise_in_place(A_groups), _pairwise_in_place(B_groups)


def forward(z: np.ndarray, y: np.ndarray, segments: int, inv_tau: float = 1.0,
            entropy: bool = False) -> dict:
    """logp, lse (and entropy) of every row from fp32 logits z [T, V] and targets y [T]."""
    z = _f32(z)
    T, V = z.shape
    tau = F(inv_tau)
    zt = z * tau if tau != F(1.0) else z
    L = V // segments
    Ms, Ss, Us = [], [], []
    for sgm in range(segments):
        m, s, u = _tile_stats(zt[:, sgm * L:(sgm + 1) * L], entropy)
        M_s, S_s, U_s = _segment_fold(m, s, u, entropy)
        Ms.append(M_s)
        Ss.append(S_s)
        Us.append(U_s)
    M = Ms[0]
    for M_s in Ms[1:]:
        M = np.maximum(M, M_s)
    a_s, a_u = [], []
    for M_s, S_s, U_s in zip(Ms, Ss, Us):
        dm = M_s - M
        e = p_exp(dm)
        a_s.append(S_s * e)
        a_u.append((U_s + S_s * dm) * e)
    S = _pairwise_in_place(a_s)
    Uu = _pairwise_in_place(a_u)
    logS = p_log(S)
    lse = M + logS
    yy = np.asarray(y, dtype=np.int64)
    act = yy >= 0
    bad = yy >= V
    zy = zt[np.arange(T), np.clip(yy, 0, V - 1)]
    out = {"logp": (zy - lse).astype(F), "lse": lse.astype(F)}
    if entropy:
        out["entropy"] = (logS - Uu / S).astype(F)
    for k in out:
        out[k] = np.where(act, out[k], F(0.0)).astype(F)
        out[k] = np.where(bad, F(np.nan), out[k]).astype(F)
    return out
