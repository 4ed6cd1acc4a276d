"""The C-ABI library on the host: it loads, exports every declared symbol, and its host-only
logic (validation, layout planning, workspace sizing, fail-closed creation) behaves. No GPU."""

import ctypes
import subprocess

import pytest
import torch

from invariant_lm_head_deterministic_amd import _lib
from invariant_lm_head_deterministic_amd import make_config, make_layout


def test_exports_every_declared_symbol(lib):
    declared = _lib.header_functions()
    assert len(declared) >= 13
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    for f in declared:
        assert hasattr(lib, f)


def test_status_strings_and_fingerprint(lib):
    for s in range(9):
        assert _lib.rlk_status_string(s) != "unknown status"
    assert _lib.rlk_status_string(99) == "unknown status"
    fp = _lib.rlk_build_fingerprint()
    assert "gfx950" in fp and "-ffp-contract=off" in fp and "-packed-fp32-ops" in fp


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_create_fails_closed_without_a_device(lib):
    with pytest.raises(_lib.RlkError) as e:
        _lib.rlk_logprob_create(make_config(4096, 151936), 0)
    assert e.value.status == _lib.RLK_ERR_NO_DEVICE


def _ws(cfg, layout):
    return _lib.rlk_logprob_workspace_size(cfg, layout)


def test_workspace_size_matches_the_partial_arrays(lib):
    cfg = make_config(4096, 151936)
    layout, _k = make_layout(4096)
    n = _ws(cfg, layout)
    tiles = 4 * 594  # 37984 = 593 * 64 + 32
    want = 256 + 4096 * 4 + 2 * tiles * 4096 * 4 + 4 * 4096 * 16
    assert want <= n <= want + 8 * 256
    cfg_e = make_config(4096, 151936, entropy=True)
    assert _ws(cfg_e, layout) >= n + tiles * 4096 * 4
    cfg_r = make_config(5120, 151936, rmsnorm=True, entropy=True, temperature=0.7)
    assert _ws(cfg_r, layout) >= _ws(make_config(5120, 151936, entropy=True), layout) + 4096 * 5120 * 2
    # the layout does not change the workspace (it is sized by rows and tiles)
    l2, _k2 = make_layout(4096, batch_sizes=[1000, 3096], row_chunk=512, vocab_shards=4)
    assert _ws(cfg, l2) == n


def test_layout_check_counts_launches(lib):
    cfg = make_config(256, 1000)
    l, _k = make_layout(64)
    assert _lib.rlk_layout_check(cfg, l) == 1
    l, _k = make_layout(64, batch_sizes=[8, 8, 16, 16, 4, 4, 4, 4])
    assert _lib.rlk_layout_check(cfg, l) == 8
    l, _k = make_layout(64, batch_sizes=[8, 8, 16, 16, 4, 4, 4, 4], vocab_shards=4)
    assert _lib.rlk_layout_check(cfg, l) == 32
    l, _k = make_layout(55296, row_chunk=2048)
    assert _lib.rlk_layout_check(make_config(4096, 151936), l) == 27
    l, _k = make_layout(55296, row_chunk=8192, vocab_shards=2)
    assert _lib.rlk_layout_check(make_config(4096, 151936), l) == 14


@pytest.mark.parametrize("kw,status", [
    (dict(hidden_size=100, vocab_size=1000), _lib.RLK_ERR_UNSUPPORTED_SHAPE),
    (dict(hidden_size=192, vocab_size=1000), _lib.RLK_ERR_UNSUPPORTED_SHAPE),
    (dict(hidden_size=256, vocab_size=1001), _lib.RLK_ERR_UNSUPPORTED_SHAPE),
    (dict(hidden_size=256, vocab_size=1000, vocab_segments=3), _lib.RLK_ERR_UNSUPPORTED_SHAPE),
    (dict(hidden_size=256, vocab_size=1000, vocab_segments=16), _lib.RLK_ERR_UNSUPPORTED_SHAPE),
    (dict(hidden_size=0, vocab_size=1000), _lib.RLK_ERR_UNSUPPORTED_SHAPE),
    # a segment longer than the fold's 128 groups of 32 tiles of 64 columns
    (dict(hidden_size=128, vocab_size=262145 * 2, vocab_segments=2), _lib.RLK_ERR_UNSUPPORTED_SHAPE),
])
def test_bad_configs_are_rejected(lib, kw, status):
    cfg = make_config(**kw)
    l, _k = make_layout(8)
    with pytest.raises(_lib.RlkError) as e:
        _ws(cfg, l)
    assert e.value.status == status
    assert _lib.rlk_last_error() != ""


def test_bad_layouts_are_rejected(lib):
    cfg = make_config(256, 1000)
    l, _k = make_layout(64, vocab_shards=3)
    with pytest.raises(_lib.RlkError) as e:
        _ws(cfg, l)
    assert e.value.status == _lib.RLK_ERR_CONTRACT
    l, _k = make_layout(64, batch_sizes=[10, 10])  # sums to 20, not 64
    with pytest.raises(_lib.RlkError) as e:
        _ws(cfg, l)
    assert e.value.status == _lib.RLK_ERR_INVALID_ARGUMENT
    l, _k = make_layout(64, token_tile=48)
    with pytest.raises(_lib.RlkError) as e:
        _ws(cfg, l)
    assert e.value.status == _lib.RLK_ERR_UNSUPPORTED_SHAPE
    l, _k = make_layout(64)
    l.reserved = 1
    with pytest.raises(_lib.RlkError):
        _ws(cfg, l)


def test_temperature_and_nan_config(lib):
    bad = make_config(256, 1000)
    bad.inv_temperature = float("nan")
    l, _k = make_layout(8)
    with pytest.raises(_lib.RlkError) as e:
        _ws(bad, l)
    assert e.value.status == _lib.RLK_ERR_INVALID_ARGUMENT
    c = make_config(256, 1000, temperature=0.7)
    assert ctypes.c_float(c.inv_temperature).value == pytest.approx(1 / 0.7, rel=1e-7)


def test_longest_segment_is_accepted(lib):
    cfg = make_config(128, 262144 * 4, vocab_segments=4)
    l, _k = make_layout(8)
    assert _ws(cfg, l) > 0


def test_fingerprint_names_the_contract_version(lib):
    # pinned on purpose: a change of the numeric contract must show up here
    import re

    fp = _lib.rlk_build_fingerprint()
    m = re.search(r"contract v(\d+)", fp)
    assert m and int(m.group(1)) == 3, fp


def test_partials_range_must_sit_on_segment_boundaries(lib):
    cfg = make_config(4096, 151936)
    assert _lib.rlk_logprob_partials_workspace_size(cfg, 128, 37984, 2 * 37984) > 0
    with pytest.raises(_lib.RlkError) as e:
        _lib.rlk_logprob_partials_workspace_size(cfg, 128, 100, 37984)
    assert e.value.status == _lib.RLK_ERR_CONTRACT


def test_flag_bits(lib):
    l, _k = make_layout(8)
    base = _ws(make_config(256, 1000, entropy=True), l)
    port = make_config(256, 1000, entropy=True, rmsnorm=True, portable=True)
    assert port.flags == (_lib.RLK_FLAG_ENTROPY | _lib.RLK_FLAG_RMSNORM
                          | _lib.RLK_FLAG_PORTABLE_EXP)
    assert _ws(make_config(256, 1000, entropy=True, portable=True), l) == base
    assert _ws(port, l) >= base
    bad = make_config(256, 1000)
    bad.flags = 8
    with pytest.raises(_lib.RlkError) as e:
        _ws(bad, l)
    assert e.value.status == _lib.RLK_ERR_INVALID_ARGUMENT


def test_backward_workspace_size(lib):
    cfg = make_config(4096, 151936, vocab_segments=4)
    n = _lib.rlk_logprob_backward_workspace_size(cfg, 4096, 0)
    Lp = 38016  # 37984 rounded up to 128
    J = 4 * Lp
    want = 4096 * J * 2 + 4 * 4096 * 4096 * 4  # dz rows, per-segment dh partials
    assert want <= n < want + 2 * 256
    m = _lib.rlk_logprob_backward_workspace_size(cfg, 4096, 1024)
    assert 1024 * J * 2 + 4 * 1024 * 4096 * 4 <= m < n
    # long batches are chunked so that a chunk's dz stays under 2 GiB: 7040 rows here
    big = _lib.rlk_logprob_backward_workspace_size(cfg, 55296, 0)
    assert 7040 * J * 2 <= big < 7040 * J * 2 + 4 * 7040 * 4096 * 4 + 2 * 256
    for bad in (100, -128):
        with pytest.raises(_lib.RlkError) as e:
            _lib.rlk_logprob_backward_workspace_size(cfg, 4096, bad)
        assert e.value.status in (_lib.RLK_ERR_UNSUPPORTED_SHAPE, _lib.RLK_ERR_INVALID_ARGUMENT)
    with pytest.raises(_lib.RlkError):
        _lib.rlk_logprob_backward_workspace_size(cfg, -1, 0)


def test_backward_shard_workspace_sizes(lib):
    cfg = make_config(256, 1000, vocab_segments=4)  # segments of 250 (padded to 256)
    n = _lib.rlk_logprob_backward_partials_workspace_size(cfg, 64, 250, 750, 0)
    assert n >= 64 * 2 * 256 * 2  # dz for the shard's 2 segments
    full = _lib.rlk_logprob_backward_workspace_size(cfg, 64, 0)
    assert n < full  # no tree partials, half the positions
    for lo, hi in ((0, 100), (250, 251), (-250, 250), (750, 1250), (500, 500)):
        with pytest.raises(_lib.RlkError) as e:
            _lib.rlk_logprob_backward_partials_workspace_size(cfg, 64, lo, hi, 0)
        assert e.value.status == _lib.RLK_ERR_CONTRACT
    assert _lib.rlk_logprob_backward_merge_workspace_size(cfg, 64) == 256
    rms = make_config(256, 1000, rmsnorm=True)
    assert _lib.rlk_logprob_backward_merge_workspace_size(rms, 64) >= 64 * 256 * 4
