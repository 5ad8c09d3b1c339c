"""Host logic of the prefix-hash index: the chained FNV-1a hashes against the published FNV-1a
definition and its reference vectors, the chain's dependence on the prefix, and argument
checks of the cache calls (no GPU work)."""
import ctypes

import numpy as np
import pytest

from cross_model_attention_amd import _lib

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    """FNV-1a 64-bit from its published definition: for each byte, xor then multiply mod 2^64."""
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & 0xFFFFFFFFFFFFFFFF
    return h


def chain(tokens: np.ndarray, B: int) -> list[int]:
    h = fnv1a64(int(B).to_bytes(4, "little"))
    out = []
    for r in range(len(tokens) // B):
        h = fnv1a64(h.to_bytes(8, "little") + tokens[r * B:(r + 1) * B].astype("<i4").tobytes())
        out.append(h)
    return out


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_fnv1a64_reference_vectors():
    # published FNV-1a 64-bit test values
    assert fnv1a64(b"") == 0xCBF29CE484222325
    assert fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert fnv1a64(b"foobar") == 0x85944171F73967E8


def _hashes(tokens, B):
    import cross_model_attention_amd as mf
    return [int(x) for x in mf.prefix_hashes(tokens, B)]


@pytest.mark.parametrize("n,B", [(0, 64), (63, 64), (64, 64), (300, 64), (257, 32), (17, 16)])
def test_prefix_hashes_follow_the_definition(n, B):
    tok = np.random.default_rng(n + B).integers(-2**31, 2**31 - 1, size=n, dtype=np.int64).astype(np.int32)
    assert _hashes(tok, B) == chain(tok, B)


def test_prefix_hash_chain_depends_on_the_whole_prefix():
    rng = np.random.default_rng(5)
    tok = rng.integers(0, 50000, size=64 * 6, dtype=np.int32)
    base = _hashes(tok, 64)
    assert len(set(base)) == 6
    for k in range(6):
        t2 = tok.copy()
        t2[64 * k + 17] += 1
        h2 = _hashes(t2, 64)
        assert h2[:k] == base[:k]                                  # rows before the change agree
        assert all(a != b for a, b in zip(h2[k:], base[k:]))       # every later row differs
    assert _hashes(tok, 32)[1] != base[0]                          # same 64 tokens, other block size
    assert _hashes(np.concatenate([tok, tok[:10]]), 64) == base    # a partial block adds no hash


def test_cache_calls_reject_bad_arguments(lib):
    out = ctypes.c_void_p()
    assert lib.mf_cache_create(None, 1 << 20, ctypes.byref(out)) == _lib.MF_ERR_INVALID
    assert lib.mf_cache_info(None, None, None) == _lib.MF_ERR_INVALID
    rows = ctypes.c_int32(0)
    assert lib.mf_cache_lookup(None, 0, None, 0, 64, ctypes.byref(rows), ctypes.byref(_lib.MfBsr())) == _lib.MF_ERR_INVALID
    assert lib.mf_cache_insert(None, 0, None, 0, 1, ctypes.byref(_lib.MfBsr()), 1, None) == _lib.MF_ERR_INVALID
    assert lib.mf_cache_destroy(None) == _lib.MF_OK
    assert lib.mf_prefix_hashes(None, 128, 64, None) == _lib.MF_ERR_INVALID
    assert lib.mf_prefix_hashes(None, 10, 0, None) == _lib.MF_ERR_INVALID
