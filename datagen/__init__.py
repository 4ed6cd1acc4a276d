"""Seeded synthetic inputs for the selected-token logprob path.

This module makes the bytes that both the HIP library and the CPU oracle are fed. It holds none
of the method's arithmetic: no logits, no softmax, no reductions. It only draws random numbers,
encodes them as bfloat16 bit patterns, and builds row layouts (ragged batch sizes, padding masks).
Values the method itself would draw (the per-row uniforms used to sample targets) are handed out
here as plain inputs; turning them into target tokens is the oracle's job (tests/golden/).

Every stream is ``numpy.random.default_rng([1234, cfg, tensor_id, chunk])``: the seed 1234 is the
training/rollout seed of the MI300X validation run on the RL-Kernel v0.1.0 summary page ("AMD
Instinct MI300X validation") and on the aihirek.info report ("200 lépésen át nulla eltérés").
Large tensors are drawn in fixed chunks of ``CHUNK`` elements, one substream per chunk, so the
bytes do not depend on how many threads draw them.
"""

from __future__ import annotations

import hashlib
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

SEED = 1234
CHUNK = 1 << 22  # elements per independent substream

# tensor ids of the substreams
TID_HIDDEN, TID_W, TID_TARGETS, TID_LAYOUT, TID_MASK, TID_GAMMA = 0, 1, 2, 3, 4, 5


def rng(cfg: int, tid: int, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng([SEED, cfg, tid, chunk])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Encode float32 values as bfloat16 bit patterns, rounding to nearest, ties to even.

    Inputs here are finite draws; NaN/Inf encodings are not needed and not special-cased.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_bf16(n_rows: int, n_cols: int, cfg: int, tid: int, scale: float = 1.0,
                mean: float = 0.0) -> np.ndarray:
    """bf16 bits of fl32(mean + fl32(scale) * N(0,1)) in a [n_rows, n_cols] uint16 array.

    The N(0,1) draw is float32; ``scale`` is rounded to float32 once; one multiply and (if
    ``mean`` is nonzero) one add in float32, then one round-to-nearest-even to bf16.
    """
    total = n_rows * n_cols
    out = np.empty(total, dtype=np.uint16)
    s32 = np.float32(scale)
    m32 = np.float32(mean)
    n_chunks = (total + CHUNK - 1) // CHUNK

    def work(c: int) -> None:
        lo = c * CHUNK
        hi = min(total, lo + CHUNK)
        x = rng(cfg, tid, c).standard_normal(hi - lo, dtype=np.float32)
        x *= s32
        if mean != 0.0:
            x += m32
        out[lo:hi] = f32_to_bf16_bits(x)

    if n_chunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(n_chunks)))
    return out.reshape(n_rows, n_cols)


def uniform_targets(n: int, vocab: int, cfg: int) -> np.ndarray:
    """Targets drawn uniformly from [0, vocab) (the tiny workload's recipe)."""
    return rng(cfg, TID_TARGETS).integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def target_uniforms(n: int, cfg: int) -> np.ndarray:
    """Per-row U[0,1) draws (float64) from which targets are sampled by inverse CDF."""
    return rng(cfg, TID_TARGETS).random(n)


def ragged_sizes_exact_sum(n_batches: int, lo: int, hi: int, total: int, cfg: int) -> list[int]:
    """n_batches iid U{lo..hi} sizes, the whole draw repeated until they sum to ``total``."""
    g = rng(cfg, TID_LAYOUT)
    for _ in range(100000):
        s = g.integers(lo, hi + 1, size=n_batches)
        if int(s.sum()) == total:
            return [int(v) for v in s]
    raise RuntimeError("no ragged draw summed to the total")


def ragged_sizes_cover(total: int, lo: int, hi: int, cfg: int, tid: int = TID_LAYOUT) -> list[int]:
    """iid U{lo..hi} sizes until the running sum reaches ``total``; the last one is truncated."""
    g = rng(cfg, tid)
    sizes: list[int] = []
    acc = 0
    while acc < total:
        s = int(g.integers(lo, hi + 1))
        s = min(s, total - acc)
        sizes.append(s)
        acc += s
    return sizes


def offsets(sizes: list[int]) -> list[int]:
    out = [0]
    for s in sizes:
        out.append(out[-1] + s)
    return out


def trailing_pad_mask(n_samples: int, sample_len: int, n_pad: int, cfg: int) -> np.ndarray:
    """Bool [n_samples*sample_len]: True where the row is padding.

    ``n_pad`` padded rows are split over the samples by one multinomial draw and placed at the
    end of each sample (responses shorter than the padded length).
    """
    counts = rng(cfg, TID_MASK).multinomial(n_pad, [1.0 / n_samples] * n_samples)
    mask = np.zeros((n_samples, sample_len), dtype=bool)
    for i, c in enumerate(counts):
        c = int(min(c, sample_len))
        if c:
            mask[i, sample_len - c:] = True
    return mask.reshape(-1)


def sha256(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).view(np.uint8).data)
    return h.hexdigest()


# --------------------------------------------------------------------------------------------
# The five workloads. Shapes follow the Qwen3-8B LM head (H=4096, V=151936) of the MI300X
# validation run, responses of up to 6912 tokens and 8 samples per prompt (aihirek.info report,
# "200 lépésen át nulla eltérés"), and a TP4 vocab partition (RL-Kernel v0.1.0 summary, the
# strict-path boundary table, row "Linear logprob").
# --------------------------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    cfg: int
    T: int
    H: int
    V: int
    hidden_scale: float
    w_scale: float = 0.02
    tau: float = 1.0
    rmsnorm: bool = False
    rms_eps: float = 1e-6
    gamma_mean: float = 1.0
    gamma_scale: float = 0.1
    w_cfg: int | None = None     # draw W from another workload's stream (same bytes)
    hidden_cfg: int | None = None
    targets: str = "softmax"      # "uniform" or "softmax" (sampled by the oracle, stored)
    segments: int = 4
    extra: dict = field(default_factory=dict)


WORKLOADS: dict[str, Workload] = {
    "tiny": Workload("tiny", 1, T=64, H=256, V=1000, hidden_scale=1.0, targets="uniform"),
    "qwen3_8b_head": Workload("qwen3_8b_head", 2, T=4096, H=4096, V=151936,
                              hidden_scale=4.0 / math.sqrt(4096)),
    "tp4_shards": Workload("tp4_shards", 3, T=4096, H=4096, V=151936,
                           hidden_scale=4.0 / math.sqrt(4096), w_cfg=2, hidden_cfg=2),
    "long_grpo": Workload("long_grpo", 4, T=55296, H=4096, V=151936,
                          hidden_scale=4.0 / math.sqrt(4096), w_cfg=2,
                          extra={"n_samples": 8, "sample_len": 6912, "n_pad": 553}),
    "norm_head": Workload("norm_head", 5, T=8192, H=5120, V=151936, hidden_scale=1.0,
                          tau=0.7, rmsnorm=True),
}


def hidden_bits(w: Workload, rows: int | None = None) -> np.ndarray:
    cfg = w.hidden_cfg if w.hidden_cfg is not None else w.cfg
    return normal_bf16(w.T if rows is None else rows, w.H, cfg, TID_HIDDEN, scale=w.hidden_scale)


def weight_bits(w: Workload) -> np.ndarray:
    cfg = w.w_cfg if w.w_cfg is not None else w.cfg
    return normal_bf16(w.V, w.H, cfg, TID_W, scale=w.w_scale)


def gamma_bits(w: Workload) -> np.ndarray:
    return normal_bf16(1, w.H, w.cfg, TID_GAMMA, scale=w.gamma_scale, mean=w.gamma_mean)[0]


def pad_mask(w: Workload) -> np.ndarray:
    if "n_pad" not in w.extra:
        return np.zeros(w.T, dtype=bool)
    e = w.extra
    return trailing_pad_mask(e["n_samples"], e["sample_len"], e["n_pad"], w.cfg)


def tiny_layout() -> list[int]:
    """Rollout layout of the tiny workload: 8 ragged batches of 1..16 rows summing to 64."""
    return ragged_sizes_exact_sum(8, 1, 16, 64, WORKLOADS["tiny"].cfg)


def decode_layout(total: int = 4096) -> list[int]:
    """Rollout layout of the TP4 workload: decode batches of U{1..256} rows covering ``total``."""
    return ragged_sizes_cover(total, 1, 256, WORKLOADS["tp4_shards"].cfg)


def dyadic_bf16(n_rows: int, n_cols: int, cfg: int, tid: int, k_max: int, log2_den: int,
                density: float = 1.0) -> np.ndarray:
    """bf16 bits of k * 2^-log2_den, k uniform on -k_max..k_max (zero where a uniform draw
    exceeds ``density``). With |k| <= 127 every value is exact in bf16, and products and sums
    of such values stay on a known dyadic grid, which lets a test reason about exactness.
    """
    assert 0 < k_max <= 127
    g = rng(cfg, tid)
    k = g.integers(-k_max, k_max + 1, size=(n_rows, n_cols), dtype=np.int8)
    if density < 1.0:
        k[g.random(size=(n_rows, n_cols), dtype=np.float32) >= density] = 0
    table = f32_to_bf16_bits(np.ldexp(np.arange(-k_max, k_max + 1, dtype=np.float64),
                                      -log2_den).astype(np.float32))
    return table[k.astype(np.int16) + k_max]


def small_case(T: int, H: int, V: int, seed_cfg: int, hidden_scale: float = 1.0,
               w_scale: float = 0.02) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """A parity case of arbitrary shape: bf16 hidden, bf16 W, uniform int32 targets.

    ``seed_cfg`` should be >= 100 so it never collides with the five workloads' streams.
    """
    h = normal_bf16(T, H, seed_cfg, TID_HIDDEN, scale=hidden_scale)
    W = normal_bf16(V, H, seed_cfg, TID_W, scale=w_scale)
    y = uniform_targets(T, V, seed_cfg)
    return h, W, y
