"""CPU checks of libsn.so: it loads, exports every declared entry point, and
its host-side helpers (parameter layout, int16 quantisation, workspace size)
behave.  No GPU work is launched here."""
import os
import re

import numpy as np
import pytest

import oracle as O
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sn():
    import schnet_cfconv_force_amd as sn
    if not os.path.exists(sn.LIB_PATH):
        from schnet_cfconv_force_amd import build
        build.build(verbose=False)       # hipcc cross-compiles without a GPU
    return sn


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "sn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sn_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    sn = _sn()
    lib = sn.lib()
    names = declared_symbols()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(sn.EXPORTED)
    assert lib.sn_version() == 3


def test_status_strings():
    sn = _sn()
    for code in range(0, -8, -1):
        assert sn.status_string(code) != "unknown status"
    assert sn.status_string(-99) == "unknown status"


@pytest.mark.parametrize("name", ["tiny_chain", "single_protein", "larger_cg", "dense_box"])
def test_param_layout_matches_shapes(name):
    sn = _sn()
    cfg = synth.make_config(name)
    h = cfg["hyper"]
    off = sn.param_offsets(h["n_types"], h["n_interactions"], h["n_features"], h["n_rbf"])
    assert len(off) == 9 * h["n_interactions"] + 6
    packed = sn.pack_params(cfg["params"], h)
    assert packed.size == off[-1] == sn.lib().sn_param_count(h["n_types"], h["n_interactions"],
                                                               h["n_features"], h["n_rbf"])
    blk = cfg["params"]["interactions"][-1]
    k = 1 + 9 * (h["n_interactions"] - 1)
    assert np.array_equal(packed[off[k + 3]:off[k + 4]], blk["A2"].ravel())
    assert packed[off[-2]] == np.float32(cfg["params"]["c2"])
    assert sn.lib().sn_param_offsets(0, 1, 32, 16, None, 0) == -1


@pytest.mark.parametrize("name", ["tiny_chain", "single_protein", "dense_box"])
def test_host_quantisation_is_bit_exact_with_oracle(name):
    sn = _sn()
    cfg = synth.make_config(name)
    h = cfg["hyper"]
    q, s = sn.quantize_filter_weights(sn.pack_params(cfg["params"], h), h)
    F, K = h["n_features"], h["n_rbf"]
    per = K * F + F * F
    for t, blk in enumerate(cfg["params"]["interactions"]):
        q1, s1 = O.quantize_per_out_channel(blk["A1"])
        q2, s2 = O.quantize_per_out_channel(blk["A2"])
        assert np.array_equal(q[per * t:per * t + K * F].reshape(K, F), q1)
        assert np.array_equal(q[per * t + K * F:per * (t + 1)].reshape(F, F), q2)
        assert np.array_equal(s[2 * F * t:2 * F * t + F], s1)
        assert np.array_equal(s[2 * F * t + F:2 * F * (t + 1)], s2)


def test_host_quantisation_hand_example_and_zero_column():
    sn = _sn()
    import json
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "quantize_hand.json")))
    T, I, F, K = 1, 1, 32, 3
    p = synth.init_params(T, I, F, K, 0)
    w = np.zeros((K, F), np.float32)
    w[:, :3] = np.array(gold["w"], np.float32)
    p["interactions"][0]["A1"] = w
    hyper = {"n_types": T, "n_interactions": I, "n_features": F, "n_rbf": K}
    q, s = sn.quantize_filter_weights(sn.pack_params(p, hyper), hyper)
    qa1 = q[:K * F].reshape(K, F)
    assert qa1[:, :3].tolist() == gold["q"]
    assert np.all(qa1[:, 3:] == 0) and np.all(s[3:F] == 0)


def test_workspace_bytes_grow_with_edges():
    sn = _sn()
    import ctypes
    cfg = synth.make_config("single_protein")
    h = cfg["hyper"]
    m = sn.binding.SnModel(h["n_types"], h["n_interactions"], h["n_features"], h["n_rbf"], h["cutoff"],
                           h["rbf_lo"], h["rbf_hi"], h["rbf_gamma"], 0, 1, None, None)
    sysc = sn.binding.SnSystem(269, 1, 1, 1, 0, (ctypes.c_float * 3)(0, 0, 0))
    a = sn.lib().sn_workspace_bytes(ctypes.byref(m), ctypes.byref(sysc), 1000)
    b = sn.lib().sn_workspace_bytes(ctypes.byref(m), ctypes.byref(sysc), 100000)
    # the stored filter rows alone need I * (E/2) * F * 3 bytes (24-bit values)
    assert b - a >= 3 * (50000 - 500) * 128 * 3
    assert sn.lib().sn_workspace_bytes(None, ctypes.byref(sysc), 0) > 0


def test_verlet_rejects_bad_schedule_and_flags_before_any_gpu_work():
    """sn_verlet_step validates rebuild_every (>= 0) and flags (0 or SN_MD_GRAPH) on the host: with
    either out of range it returns SN_ERR_INVALID before touching a pointer (the ones passed here are
    dummies that a GPU call would fault on)."""
    sn = _sn()
    import ctypes
    cfg = synth.make_config("tiny_chain")
    h = cfg["hyper"]
    m = sn.binding.SnModel(h["n_types"], h["n_interactions"], h["n_features"], h["n_rbf"], h["cutoff"],
                           h["rbf_lo"], h["rbf_hi"], h["rbf_gamma"], 0, 16, None, None)
    sysc = sn.binding.SnSystem(32, 1, 16, 16, 0, (ctypes.c_float * 3)(0, 0, 0))
    lib = sn.lib()
    ne = ctypes.c_int64(0)
    done = ctypes.c_int32(7)
    dummy = 16

    def call(n_steps, rebuild_every, flags, r_list=11.0):
        return lib.sn_verlet_step(ctypes.byref(m), ctypes.byref(sysc), dummy, dummy, dummy, dummy, 2.0,
                                  synth.FORCE_TO_ACCEL, n_steps, rebuild_every, r_list, dummy, dummy, dummy, 1000,
                                  ctypes.byref(ne), None, None, None, ctypes.byref(done), flags, dummy, 1 << 30,
                                  None)
    assert call(10, -1, 0) == sn.SN_ERR_INVALID
    assert done.value == 0                       # written before any check
    assert call(10, 5, 2) == sn.SN_ERR_INVALID   # unknown flag bit
    assert call(10, 5, sn.SN_MD_GRAPH | 4) == sn.SN_ERR_INVALID
    assert call(-1, 1, 0) == sn.SN_ERR_INVALID
    assert call(10, 1, 0, r_list=float("nan")) == sn.SN_ERR_INVALID
    # the filter arithmetic is 0 (fp32-accurate) or 1 (one fp16 product); others are refused
    m.filter_math = 2
    assert call(10, 1, 0) == sn.SN_ERR_INVALID
    m.filter_math = -1
    assert call(10, 1, 0) == sn.SN_ERR_INVALID
