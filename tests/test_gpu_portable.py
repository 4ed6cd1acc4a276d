"""The portable mode (software EXP, LOG and RSQ) reproduces, bit for bit, a float32 CPU model of
the numeric contract written independently of the HIP code (tests/contract_f32.py).

Inputs are dyadic (small integers times powers of two) so that the logits are exact in fp32
whatever the GEMM's summation order; from the logits on, every step of the contract is an IEEE
fp32 operation the CPU performs identically. The pages ask that a forward's primitives and
reduction orders be fixed so that independent executions agree exactly (RL-Kernel v0.1.0 summary
page, "Numeric execution contract"; nxbn.cn blog, section 4.4: equality, not a tolerance).
"""

import numpy as np
import pytest

import datagen
import oracle
from tests import contract_f32 as cf
from tests.helpers import assert_bitwise, dev_bits, dev_i32, diff_stats, host, say

pytestmark = pytest.mark.gpu


def _dyadic(T, H, V, cfg):
    h = datagen.dyadic_bf16(T, H, cfg, datagen.TID_HIDDEN, k_max=4, log2_den=2)
    W = datagen.dyadic_bf16(V, H, cfg, datagen.TID_W, k_max=4, log2_den=4)
    y = datagen.uniform_targets(T, V, cfg)
    return h, W, y


def _inv_tau(tau):
    return float(np.float32(1.0 / tau))


def _keys(ent):
    return ("logp", "lse", "entropy") if ent else ("logp", "lse")


def _check_model(got, want, keys, what):
    for k in keys:
        assert_bitwise(host(got[k]) if not isinstance(got[k], np.ndarray) else got[k], want[k],
                       f"{what} {k}")


CASES = [
    # T, H, V, S_c, tau, entropy, layout
    (300, 256, 5000, 4, 1.0, True, {}),                  # > 256 rows: the 256x256 kernel
    (300, 256, 5000, 4, 0.7, False, {}),                 # temperature
    (200, 512, 3000, 2, 1.0, True, {}),                  # 193..256 rows: decode kernels
    (150, 256, 4000, 4, 1.0, False, {}),                 # 129..192 rows
    (77, 384, 2048, 4, 1.0, True, {}),                   # 65..128 rows, whole tiles only
    (20, 128, 9000, 1, 1.0, True, {}),                   # one segment of 141 tiles: 5 fold groups
    (512, 256, 5000, 4, 0.7, True, {}),                  # whole row tiles (2 x 256)
    (16, 512, 3000, 4, 0.7, True, {}),                   # <= 16 rows: streaming kernel, 256-K stages
    (29, 384, 3000, 2, 1.0, True, {}),                   # 17..32 rows: 2 compute waves, 128-K stages
    (5, 256, 2600, 4, 1.0, False, {}),                   # streaming kernel, one 256-K stage per tile
    (9, 256, 5600, 8, 0.7, True, {}),                    # 8 segments of 700
    (29, 512, 3000, 2, 0.7, True, {}),                   # 17..32 rows: interleaved 3-tile kernel
    (60, 256, 5000, 4, 1.0, True, {}),                   # 33..64 rows, last item of 2 tiles
    (100, 768, 2500, 1, 0.7, False, {}),                 # 65..128 rows, 3 K chunks
    (300, 256, 5000, 4, 1.0, True, {"token_tile": 32}),
    (300, 256, 5000, 4, 1.0, True, {"token_tile": 64}),
    (300, 256, 5000, 4, 1.0, True, {"token_tile": 128}),
    (130, 256, 5000, 4, 1.0, True, {"token_tile": 256}),
]


@pytest.mark.parametrize("T,H,V,S,tau,ent,lay", CASES)
def test_portable_equals_cpu_model(rlk, T, H, V, S, tau, ent, lay):
    import torch

    h, W, y = _dyadic(T, H, V, 400 + T + S)
    y[::7] = -1
    say(f"portable T={T} H={H} V={V} S={S} tau={tau} ent={ent} {lay}")
    lp = rlk.Logprob(H, V, vocab_segments=S, temperature=tau, entropy=ent, portable=True)
    got = lp.forward(dev_bits(h), dev_bits(W), dev_i32(y), **lay)
    torch.cuda.synchronize()
    want = cf.forward(cf.exact_logits(h, W), y, S, inv_tau=_inv_tau(tau), entropy=ent)
    _check_model(got, want, _keys(ent), "forward")


def test_portable_layouts_and_shard_merge_equal_cpu_model(rlk):
    import torch

    T, H, V, S = 500, 256, 8 * 777, 8
    h, W, y = _dyadic(T, H, V, 451)
    y[::9] = -1
    want = cf.forward(cf.exact_logits(h, W), y, S, entropy=True)
    lp = rlk.Logprob(H, V, vocab_segments=S, entropy=True, portable=True)
    ragged = datagen.ragged_sizes_cover(T, 1, 256, 451)
    hd, Wd, yd = dev_bits(h), dev_bits(W), dev_i32(y)
    for lay in (dict(batch_sizes=ragged), dict(vocab_shards=4), dict(row_chunk=37),
                dict(batch_sizes=ragged, vocab_shards=2, token_tile=32)):
        say(f"portable layout {lay}")
        got = lp.forward(hd, Wd, yd, **lay)
        torch.cuda.synchronize()
        _check_model(got, want, _keys(True), str(lay))
    say("portable partials over 2 shards + merge")
    seg = V // S
    recs = torch.empty((S, T, 4), dtype=torch.float32, device="cuda")
    for v0, v1 in ((0, 3 * seg), (3 * seg, V)):
        lp.partials(hd, Wd[v0:v1], v0, v1, yd, records=recs[v0 // seg:v1 // seg])
    got = lp.merge(recs, yd)
    torch.cuda.synchronize()
    _check_model(got, want, _keys(True), "partials+merge")


def test_portable_rmsnorm_equals_cpu_model(rlk):
    import torch

    T, H, V, S = 90, 512, 3000, 4
    x = datagen.dyadic_bf16(T, H, 460, datagen.TID_HIDDEN, k_max=4, log2_den=0)
    gk = datagen.dyadic_bf16(1, H, 460, datagen.TID_GAMMA, k_max=4, log2_den=3)[0]
    g = datagen.f32_to_bf16_bits(cf.bf16_to_f32(gk) + np.float32(1.0))  # (8 + k) / 8
    W = datagen.dyadic_bf16(V, H, 460, datagen.TID_W, k_max=1, log2_den=0, density=1 / 16)
    y = datagen.uniform_targets(T, V, 460)
    eps = 1e-6
    say(f"portable rmsnorm T={T} H={H} V={V}")
    lp = rlk.Logprob(H, V, vocab_segments=S, rmsnorm=True, rms_eps=eps, entropy=True,
                     portable=True)
    got = lp.forward(dev_bits(x), dev_bits(W), dev_i32(y), gamma=dev_bits(g))
    torch.cuda.synchronize()
    hn = cf.rmsnorm_bits(x, g, eps)
    want = cf.forward(cf.exact_logits(hn, W), y, S, entropy=True)
    _check_model(got, want, _keys(True), "rmsnorm")


def test_portable_and_default_both_match_oracle(rlk):
    import torch

    T, H, V, S = 257, 512, 6000, 4
    h, W, y = datagen.small_case(T, H, V, 470)
    say("portable vs default on normal inputs")
    outs = {}
    for port in (False, True):
        lp = rlk.Logprob(H, V, vocab_segments=S, temperature=0.8, entropy=True, portable=port)
        o = lp.forward(dev_bits(h), dev_bits(W), dev_i32(y))
        torch.cuda.synchronize()
        outs[port] = ({k: host(o[k]) for k in _keys(True)}, lp.contract_id)
    assert outs[False][1] != outs[True][1]
    assert "exp=soft" in outs[True][1] and "rsq=1/sqrt" in outs[True][1]
    want = oracle.logprob(h, W, y, tau=0.8, want_entropy=True)
    for port in (False, True):
        for k in _keys(True):
            s = diff_stats(outs[port][0][k], want[k])
            print(port, k, s, flush=True)
            assert s["max"] <= 1e-3, (port, k, s)


def test_portable_full_size_sampled_rows_equal_cpu_model(rlk):
    """The Qwen3-8B head shape (T=4096, H=4096, V=151936, 4 segments) in the launch the bench
    times, on 48 sampled rows checked bit for bit (rows are independent in the contract)."""
    import torch

    T, H, V, S = 4096, 4096, 151936, 4
    h, W, y = _dyadic(T, H, V, 480)
    say(f"portable full size T={T} H={H} V={V}")
    lp = rlk.Logprob(H, V, vocab_segments=S, entropy=True, portable=True)
    got = lp.forward(dev_bits(h), dev_bits(W), dev_i32(y))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, T, 97), [T - 1, 255, 256, 2047, 2048]]))
    want = cf.forward(cf.exact_logits(h[rows], W), y[rows], S, entropy=True)
    for k in _keys(True):
        assert_bitwise(host(got[k])[rows], want[k], f"full size {k}")
