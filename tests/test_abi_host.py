"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and its host logic (config checks, weight count, flow-time schedule,
error codes) behaves as include/smolexp.h states.  No GPU needed."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import flow_matching_action_step_amd as fm
import oracle
import synth

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "smolexp.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(smolexp_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 12
    out = subprocess.run(["nm", "-D", "--defined-only", fm.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (smolexp_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(fm.raw(), n)
    assert set(fm.EXPORTED) == set(names)


def test_lm_weight_count_matches_manifest():
    for L in (1, 4, 16):
        assert fm.smolexp_lm_weight_count(fm.smolexp_default_config(n_layers=L)) == synth.lm_weight_count(L)
    assert fm.smolexp_lm_weight_count(fm.smolexp_default_config()) == 16 * 9_832_320
    bad = fm.smolexp_default_config()
    bad.head_dim = 32
    assert fm.smolexp_lm_weight_count(bad) == 0


def test_prefill_checks_arguments_before_any_launch():
    lib = fm.raw()
    assert lib.smolexp_prefill(None, None, None, 1, None, 1, None) == fm.SMOLEXP_E_INVAL
    assert lib.smolexp_load_lm_weights(None, None, 0) == fm.SMOLEXP_E_INVAL


def test_train_step_checks_arguments_before_any_launch():
    lib = fm.raw()
    assert lib.smolexp_train_step(None, None, None, 1, None, None, None, None, None, 1, None) == fm.SMOLEXP_E_INVAL
    # the binding refuses host tensors before calling the library
    import torch
    cfg = fm.smolexp_default_config(n_layers=2, max_batch=1, max_prefix=4)
    x = torch.zeros((1, 50, 32))
    with pytest.raises(ValueError):
        fm.smolexp_train_step(None, cfg, torch.zeros((2, 2, 1, 5, 4, 64), dtype=torch.int16),
                              torch.ones((1, 4), dtype=torch.uint8), x, x, torch.zeros(1),
                              torch.zeros(fm.smolexp_weight_count(cfg)), torch.zeros(1))


def test_weight_count_matches_manifest():
    for L in (1, 2, 4, 16):
        assert fm.smolexp_weight_count(fm.smolexp_default_config(n_layers=L)) == synth.weight_count(L)
    assert fm.smolexp_weight_count(fm.smolexp_default_config()) == 98_210_912


@pytest.mark.parametrize("field,value", [("d_model", 512), ("n_q_heads", 16), ("n_kv_heads", 4), ("head_dim", 128),
                                         ("ffn", 4096), ("chunk", 32), ("action_dim", 16), ("n_layers", 0),
                                         ("n_layers", 65), ("n_steps", 0), ("n_steps", 65), ("max_batch", 0),
                                         ("max_batch", 1025), ("max_prefix", 0), ("rms_eps", 0.0),
                                         ("rope_theta", -1.0), ("t_max_period", 1e-3), ("weight_format", 2),
                                         ("weight_format", -1), ("batch_groups", 9)])
def test_invalid_config_is_rejected_before_any_device_call(field, value):
    cfg = fm.smolexp_default_config(**{field: value})
    assert fm.smolexp_weight_count(cfg) == 0
    h = ctypes.c_void_p()
    assert fm.raw().smolexp_create(ctypes.byref(cfg), 0, ctypes.byref(h)) == fm.SMOLEXP_E_INVAL
    assert not h.value


def test_schedule_matches_the_oracle_bitwise():
    for n in (1, 4, 10, 64):
        ts, dt = fm.smolexp_schedule(fm.smolexp_default_config(n_steps=n))
        ots, odt = oracle.schedule(n)
        assert np.array(ts, np.float32).tobytes() == np.array(ots, np.float32).tobytes()
        assert np.float32(dt) == odt


def test_null_handle_and_error_strings():
    lib = fm.raw()
    assert lib.smolexp_denoise(None, None, None, 1, None, None, 1, None) == fm.SMOLEXP_E_INVAL
    assert lib.smolexp_denoise_ex(None, None, None, 1, None, None, 1, None, None) == fm.SMOLEXP_E_INVAL
    assert lib.smolexp_velocity(None, None, None, 1, None, 0.5, None, 1, None) == fm.SMOLEXP_E_INVAL
    assert lib.smolexp_load_weights(None, None, 0) == fm.SMOLEXP_E_INVAL
    us = ctypes.c_float()
    assert lib.smolexp_time_kernel(None, 0, 1, None, ctypes.byref(us)) == fm.SMOLEXP_E_INVAL
    assert lib.smolexp_schedule(None, None, None) == fm.SMOLEXP_E_INVAL
    assert lib.smolexp_create(None, 0, None) == fm.SMOLEXP_E_INVAL
    cfg = fm.smolexp_default_config()
    assert lib.smolexp_create(ctypes.byref(cfg), -1, ctypes.byref(ctypes.c_void_p())) == fm.SMOLEXP_E_INVAL
    assert fm.smolexp_last_error(None) == ""
    lib.smolexp_destroy(None)
    names = {fm.smolexp_strerror(c) for c in (0, -1, -2, -3, -4, -5)}
    assert len(names) == 6 and fm.smolexp_strerror(-99) == "unknown error code"


def test_create_without_a_gpu_reports_a_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    cfg = fm.smolexp_default_config()
    h = ctypes.c_void_p()
    assert fm.raw().smolexp_create(ctypes.byref(cfg), 0, ctypes.byref(h)) == fm.SMOLEXP_E_HIP
    assert not h.value


def test_eight_bit_weights_take_batches_of_at_most_eight():
    ok = fm.smolexp_default_config(weight_format=fm.SMOLEXP_WEIGHTS_E4M3, max_batch=8)
    assert fm.smolexp_weight_count(ok) == 98_210_912
    bad = fm.smolexp_default_config(weight_format=fm.SMOLEXP_WEIGHTS_E4M3)  # max_batch 128
    assert fm.smolexp_weight_count(bad) == 0
    assert fm.smolexp_weight_count(fm.smolexp_default_config(weight_format=fm.SMOLEXP_WEIGHTS_E4M3, max_batch=9)) == 0


def test_e4m3_row_quantizer_matches_the_oracle_code_for_code():
    rng = np.random.default_rng(7)
    parts = [
        rng.standard_normal((40, 96)) * 0.02,                                       # weight-like rows
        rng.standard_normal((16, 96)) * np.exp(rng.uniform(-30, 30, 16))[:, None],  # any magnitude
        np.zeros((2, 96)),                                                          # all-zero rows
    ]
    W = np.concatenate(parts)
    # rows with exact ties (midpoints between neighbouring codes after the row scale) and
    # values in the subnormal range of the codes
    W[3, :8] = [448.0, 1 + 1 / 16, 1 + 3 / 16, -(1 + 5 / 16), 0.5 * 2 ** -9, 1.5 * 2 ** -9, 7.5 * 2 ** -9, -224.0]
    W[4] = np.linspace(-448, 448, 96) * 2.0 ** -12
    W[5, 0] = -0.0
    codes, scales = fm.smolexp_quantize_e4m3_rows(W)
    oc, os_ = oracle.quant.quantize_rows(W)
    np.testing.assert_array_equal(codes, oc)
    np.testing.assert_array_equal(scales.astype(np.float64), os_)
    np.testing.assert_array_equal(fm.smolexp_quantize_e4m3_rows(np.zeros((0, 5)))[0].shape, (0, 5))


def test_e4m3_row_quantizer_rejects_what_it_cannot_encode():
    for bad in (np.array([[1.0, np.nan]]), np.array([[np.inf, 0.0]]), np.array([[1e-40, 0.0]]),
                np.array([[1e300, 1.0]])):
        with pytest.raises(fm.SmolexpError):
            fm.smolexp_quantize_e4m3_rows(bad)
    raw = fm.raw()
    assert raw.smolexp_quantize_e4m3_rows(None, 1, 1, None, None) == fm.SMOLEXP_E_INVAL
    assert raw.smolexp_quantize_e4m3_rows(None, -1, 3, None, None) == fm.SMOLEXP_E_INVAL
