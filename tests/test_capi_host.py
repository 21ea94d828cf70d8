"""The C ABI without a GPU: exported symbols, host helpers, config checks."""
import os
import re
import subprocess

import numpy as np
import pytest

from conftest import ROOT
from oracle import delay_codes, undelay_codes
from synth import CONFIGS, config

HEADER = os.path.join(ROOT, "include", "moshi.h")


@pytest.fixture(scope="module")
def fds():
    import full_duplex_speech_amd as m
    m.lib()  # raises if the library is not built
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moshi_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(fds):
    names = declared_functions()
    assert len(names) >= 13
    out = subprocess.run(["nm", "-D", "--defined-only", fds.binding.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (moshi_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(fds.binding.EXPORTS) == set(names)


@pytest.mark.parametrize("tau", [0, 1, 2, 5])
def test_delay_helpers_match_oracle(fds, tau):
    rng = np.random.default_rng(tau)
    x = rng.integers(0, 2048, size=(23, 8)).astype(np.int32)
    d = fds.moshi_delay_codes(x, tau, 2048)
    np.testing.assert_array_equal(d, delay_codes(x, tau, 2048))
    np.testing.assert_array_equal(fds.moshi_undelay_codes(d, tau), undelay_codes(d, tau))
    np.testing.assert_array_equal(fds.moshi_undelay_codes(d, tau), x[: 23 - tau])


def test_delay_helpers_edge_cases(fds):
    empty = np.zeros((0, 8), np.int32)
    assert fds.moshi_delay_codes(empty, 1, 2048).shape == (0, 8)
    assert fds.moshi_undelay_codes(np.zeros((1, 8), np.int32), 1).shape == (0, 8)
    lib = fds.lib()
    assert lib.moshi_delay_codes(None, 3, 1, 0, None) == fds.binding.MOSHI_EINVAL
    assert lib.moshi_delay_codes(None, 1, -1, 0, None) == fds.binding.MOSHI_EINVAL


@pytest.mark.parametrize("name", list(CONFIGS))
def test_presets_are_valid_and_sized(fds, name):
    cfg = CONFIGS[name]
    c = fds.config_struct(cfg)
    rc, msg = fds.moshi_check_config(c)
    assert rc == 0, msg
    nbytes = fds.moshi_workspace_bytes(c)
    assert nbytes > 0 and nbytes % 256 == 0
    # at least the weights and the KV pool
    from synth import param_count
    esz = 2 if cfg.dtype == "bf16" else 4
    assert nbytes > param_count(cfg) * esz


@pytest.mark.parametrize("field,value", [("n_heads_t", 3), ("n_q", 7), ("max_batch", 9), ("max_batch", 0),
                                         ("page_frames", 48), ("dtype", 5), ("delay", -1), ("d_t", 0),
                                         ("ffn_t", 100), ("norm_eps", 0.0)])
def test_bad_configs_rejected(fds, field, value):
    c = fds.config_struct(config("tiny"))
    setattr(c, field, value)
    rc, msg = fds.moshi_check_config(c)
    assert rc == fds.binding.MOSHI_EINVAL and msg
    assert fds.moshi_workspace_bytes(c) == 0


def test_create_rejects_bad_arguments_without_touching_the_device(fds):
    c = fds.config_struct(config("tiny"))
    with pytest.raises(fds.MoshiError) as e:
        fds.moshi_create(c, 0, 0, 0)  # null workspace
    assert e.value.code == fds.binding.MOSHI_EINVAL
    with pytest.raises(fds.MoshiError) as e:
        fds.moshi_create(c, 0, 1 << 20, 16)  # too small: rejected before any device access
    assert e.value.code == fds.binding.MOSHI_ENOMEM


def test_q8_config_rules(fds):
    """8-bit models stream one conversation and need 32-aligned linear inputs; their
    workspace adds the codes (half the bf16 weight bytes) and the block parameters."""
    cfg = config("mid_q8")
    ok = fds.config_struct(cfg, max_batch=1)
    bad = fds.config_struct(cfg, max_batch=2)
    assert fds.moshi_check_config(ok)[0] == 0
    rc, msg = fds.moshi_check_config(bad)
    assert rc != 0 and "max_batch" in msg
    bf = fds.config_struct(config("mid_bf16"), max_batch=1)
    extra = fds.moshi_workspace_bytes(ok) - fds.moshi_workspace_bytes(bf)
    assert extra > 0
