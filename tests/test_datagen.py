"""The seeded input generators: determinism, encodings and layout recipes (no GPU)."""

import numpy as np
import torch

import datagen


def test_bf16_encoding_matches_torch_rne():
    g = np.random.default_rng(2)
    x = (g.standard_normal(100000) * np.exp(g.uniform(-30, 30, 100000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(datagen.f32_to_bf16_bits(x), ref)


def test_normal_bf16_is_deterministic_and_chunk_independent():
    a = datagen.normal_bf16(3, datagen.CHUNK // 2 + 5, 101, 0, scale=0.02)
    b = datagen.normal_bf16(3, datagen.CHUNK // 2 + 5, 101, 0, scale=0.02)
    assert np.array_equal(a, b)
    # the first chunk equals a direct draw from substream 0
    direct = datagen.rng(101, 0, 0).standard_normal(datagen.CHUNK, dtype=np.float32) * np.float32(0.02)
    assert np.array_equal(a.reshape(-1)[: datagen.CHUNK], datagen.f32_to_bf16_bits(direct))


def test_normal_bf16_distribution():
    w = datagen.normal_bf16(512, 1024, 102, 1, scale=0.02)
    v = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert abs(v.mean()) < 1e-3 and abs(v.std() - 0.02) < 5e-4
    gmm = datagen.normal_bf16(1, 4096, 102, 5, scale=0.1, mean=1.0)
    gv = torch.from_numpy(gmm.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert abs(gv.mean() - 1.0) < 1e-2 and abs(gv.std() - 0.1) < 1e-2


def test_tiny_workload_bytes_are_stable():
    w = datagen.WORKLOADS["tiny"]
    h = datagen.hidden_bits(w)
    W = datagen.weight_bits(w)
    y = datagen.uniform_targets(w.T, w.V, w.cfg)
    assert h.shape == (64, 256) and W.shape == (1000, 256) and y.shape == (64,)
    assert y.min() >= 0 and y.max() < 1000
    assert datagen.sha256(h, W, y) == datagen.sha256(datagen.hidden_bits(w), datagen.weight_bits(w),
                                                     datagen.uniform_targets(w.T, w.V, w.cfg))


def test_tiny_rollout_layout():
    sizes = datagen.tiny_layout()
    assert len(sizes) == 8 and sum(sizes) == 64 and all(1 <= s <= 16 for s in sizes)


def test_decode_layout_covers_rows():
    sizes = datagen.decode_layout(4096)
    assert sum(sizes) == 4096 and all(1 <= s <= 256 for s in sizes)
    assert 20 <= len(sizes) <= 60
    offs = datagen.offsets(sizes)
    assert offs[0] == 0 and offs[-1] == 4096


def test_long_grpo_pad_mask():
    w = datagen.WORKLOADS["long_grpo"]
    m = datagen.pad_mask(w)
    assert m.shape == (55296,) and int(m.sum()) == 553
    # padding is trailing within each of the 8 samples of 6912 rows
    for s in range(8):
        seg = m[s * 6912:(s + 1) * 6912]
        n = int(seg.sum())
        assert not seg[: 6912 - n].any() and seg[6912 - n:].all()
