"""libmapflow on the CPU: the shared library loads, exports every symbol the header declares, and
its host-only logic (layer map, argument validation) behaves as documented.  No GPU calls."""
import ctypes
import os
import re

import pytest

import oracle
from cross_model_attention_amd import _lib

HEADER = _lib.HEADER


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mf_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmapflow.so is not built; run `python cross_model_attention_amd/build.py`")
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) >= 15
    for name in names:
        assert hasattr(lib, name), name
    # and the binding declares a signature for each of them
    assert set(names) == set(_lib._SIGNATURES)


def test_version(lib):
    assert lib.mf_version().decode().startswith("libmapflow")


@pytest.mark.parametrize("n_recv,n_send,R", [(28, 36, 2), (5, 5, 0), (3, 6, 0), (1, 4, 0), (40, 48, 3),
                                             (36, 28, 0), (7, 2, 1), (4, 4, 4)])
def test_map_layers_matches_oracle(lib, n_recv, n_send, R):
    out = (ctypes.c_int32 * n_recv)()
    assert lib.mf_layer_map_uniform(n_recv, n_send, R, out) == _lib.MF_OK
    assert list(out) == oracle.layer_map(n_recv, n_send, R)
    assert lib.mf_check_layer_map(out, n_recv, n_send, R) == _lib.MF_OK


def test_check_layer_map_rejects(lib):
    bad = _lib.i32_array([-1, 0, 5])
    assert lib.mf_check_layer_map(bad, 3, 5, 1) == _lib.MF_ERR_INVALID          # 5 >= n_send
    assert "outside" in lib.mf_last_error().decode()
    bad2 = _lib.i32_array([0, 1, 2])
    assert lib.mf_check_layer_map(bad2, 3, 5, 1) == _lib.MF_ERR_INVALID         # layer 0 < R
    assert lib.mf_layer_map_uniform(3, 5, 4, (ctypes.c_int32 * 3)()) == _lib.MF_ERR_INVALID
    assert lib.mf_layer_map_uniform(0, 5, 0, (ctypes.c_int32 * 1)()) == _lib.MF_ERR_INVALID
    # installing a map needs a context, and the map is checked first
    good = _lib.i32_array([-1, 0, 4])
    assert lib.mf_map_layers(None, good, 3, 5, 1) == _lib.MF_ERR_INVALID
    assert "context" in lib.mf_last_error().decode()


def test_allocator_callbacks_come_in_pairs(lib):
    # one callback without the other is an argument error, checked before any device query
    h = ctypes.c_void_p()
    a = _lib.ALLOC_FN(lambda n, s, u: None)
    assert lib.mf_create(0, a, ctypes.cast(None, _lib.FREE_FN), None, ctypes.byref(h)) == _lib.MF_ERR_INVALID
    assert "both" in lib.mf_last_error().decode()
    assert not h.value


def test_prefill_layers_rejects_before_any_gpu_work(lib):
    assert lib.mf_prefill_layers(None, None, None, 1, 8, 8, 128, None, 0.9, 1, None, 0, None, None) == \
        _lib.MF_ERR_INVALID
    assert lib.mf_prefill_timings(None, None, None, None, None) == _lib.MF_ERR_INVALID


def test_invalid_arguments_rejected_before_any_gpu_work(lib):
    raw = _lib.MfBsr()
    cu = _lib.i32_array([0, 100])
    # bad geometry is rejected on the host (no context needed to get there)
    assert lib.mf_bsr_create(None, 4, 48, cu, 1, -1, ctypes.byref(raw)) == _lib.MF_ERR_INVALID
    assert "block size" in lib.mf_last_error().decode()
    assert lib.mf_bsr_create(None, 0, 32, cu, 1, -1, ctypes.byref(raw)) == _lib.MF_ERR_INVALID
    dec = _lib.i32_array([0, 100, 50])
    assert lib.mf_bsr_create(None, 4, 32, dec, 2, -1, ctypes.byref(raw)) == _lib.MF_ERR_INVALID
    assert "non-decreasing" in lib.mf_last_error().decode()
    assert lib.mf_bsr_create(None, 4, 32, _lib.i32_array([1, 5]), 1, -1, ctypes.byref(raw)) == _lib.MF_ERR_INVALID
    # a valid geometry but no context
    assert lib.mf_bsr_create(None, 4, 32, cu, 1, -1, ctypes.byref(raw)) == _lib.MF_ERR_INVALID
    assert "context" in lib.mf_last_error().decode()
    # compress into a store that does not exist
    assert lib.mf_compress_into(None, None, None, 1, 64, 0.9, ctypes.byref(_lib.MfBsr()), None) == _lib.MF_ERR_INVALID
    # retrieve with missing pieces
    assert lib.mf_retrieve_prepared(None, ctypes.byref(_lib.MfBsr()), None, 2, None, None, None, None) == _lib.MF_ERR_INVALID
    assert lib.mf_retrieve_multi(None, ctypes.byref(_lib.MfBsr()), 1, None, None, None, None, None,
                                 None) == _lib.MF_ERR_INVALID
    assert "store" in lib.mf_last_error().decode()
    assert lib.mf_copy_probe(None, ctypes.c_void_p(16), ctypes.c_void_p(32), 15, None) == _lib.MF_ERR_INVALID
    assert lib.mf_read_probe(None, ctypes.c_void_p(16), 15, ctypes.c_void_p(64), None) == _lib.MF_ERR_INVALID
    assert lib.mf_read_probe(None, ctypes.c_void_p(16), 16, None, None) == _lib.MF_ERR_INVALID
    assert lib.mf_write_probe(None, None, 20480, None, None) == _lib.MF_ERR_INVALID
    assert lib.mf_write_probe(None, ctypes.c_void_p(16), 20480 + 16, None, None) == _lib.MF_ERR_INVALID
    assert lib.mf_write_probe(None, ctypes.c_void_p(16), 20480, ctypes.c_void_p(8), None) == _lib.MF_ERR_INVALID
    assert lib.mf_fill_probe(None, None, 262144, 0, None) == _lib.MF_ERR_INVALID
    assert lib.mf_fill_probe(None, ctypes.c_void_p(16), 262144 + 20480, 0, None) == _lib.MF_ERR_INVALID
    assert lib.mf_fill_probe(None, ctypes.c_void_p(8), 262144, 0, None) == _lib.MF_ERR_INVALID


def test_store_layout_helpers_round_trip():
    import numpy as np
    from cross_model_attention_amd.mapflow import probs_canonical_to_store, probs_store_to_canonical
    rng = np.random.default_rng(0)
    for H_s in [4, 32, 40]:
        x = rng.random((3, H_s, 8, 8)).astype(np.float32)
        x = ((x.view(np.uint32) >> 16) << 16).view(np.float32)   # bf16 values
        bits = probs_canonical_to_store(x, H_s)
        assert bits.shape == (3, (H_s + 7) // 8, 8, 8, 8)
        # element [n, h/8, r, c, h%8] is head h's value at (r, c)
        assert bits[1, 0, 2, 3, 1] == (x[1, 1, 2, 3].view(np.uint32) >> 16)
        assert np.array_equal(probs_store_to_canonical(bits, H_s), x.astype(np.float64))
